// Binarize-and-pack kernels for gfx950.
//
// Hamming Attention Distillation (abstract): queries and keys become {-1,+1}
// vectors.  BinaryAttention (section 2.2, scaled binarized representation):
// x~ = alpha * sign(x - mu), mu a mean, alpha a scale.  Reading used here:
// mu is the per-(batch, head, channel) mean over tokens and alpha the
// per-token mean |x - mu| over channels; sign(0) = +1.
//
// The pack is a streaming scan, bound by HBM bandwidth: every input byte is
// read once (twice for the mean pass) and d/8 bytes (+4 for alpha) are
// written per token.  Loads are 16-byte vectors, eight channels per lane and
// d/8 consecutive lanes per token row, so a wave reads whole rows.
#include <algorithm>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

constexpr int kThreads = 256;

template <typename T>
HAD_DEVICE void load8(const T* p, float (&v)[8]);

template <>
HAD_DEVICE void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
HAD_DEVICE void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
  v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
  v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

// One or two tensors per launch (had_pack_qk packs Q and K together): the grid
// holds `count` equal halves, and a workgroup takes the tensor of its half.
struct Sets {
  const void* x[2];
  uint32_t* bits[2];
  float* alpha[2];
  float* mu[2];
  double* partial[2];
};

// Column sums of a workgroup's rows, in float64, in one fixed order: each thread runs
// over its rows (r_off + RPP k, k ascending) for eight columns, a butterfly over the
// lanes of a wave that hold the same columns adds the runs (every lane ends with the
// same bits: each step adds the same two values, in either order), and the kWaves
// wave sums are added in wave order by the caller.  s holds the wave sums afterwards.
constexpr int kPackWaves = kThreads / 64;
template <int D>
HAD_DEVICE void wave_colsum(double (&s)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = butterfly_f64<D / 8>(s[c], [](double a, double b) { return a + b; });
}

// Column sums over one chunk of tokens, in float64: partial[bh][chunk][c].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void colsum_partial_kernel(const Sets S, int64_t n, int64_t chunks,
                                                                  int64_t per) {
  constexpr int TPR = D / 8;          // threads per token row
  constexpr int RPP = kThreads / TPR;  // rows per pass
  __shared__ double red[kPackWaves][D];
  const int set = (int)(blockIdx.x / per);
  const int64_t b = blockIdx.x % per;
  const T* __restrict__ x = static_cast<const T*>(S.x[set]);
  const int64_t bh = b / chunks;
  const int64_t chunk = b % chunks;
  const int t = threadIdx.x;
  const int r_off = t / TPR, cg = t % TPR;
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t r0 = chunk * kPackChunk;
  for (int k = 0; k < kPackChunk / RPP; ++k) {
    const int64_t r = r0 + r_off + (int64_t)RPP * k;
    if (r < n) {
      float v[8];
      load8<T>(x + (bh * n + r) * D + 8 * cg, v);
#pragma unroll
      for (int c = 0; c < 8; ++c) s[c] += (double)v[c];
    }
  }
  wave_colsum<D>(s);
  if (t % 64 < TPR) {
#pragma unroll
    for (int c = 0; c < 8; ++c) red[t / 64][8 * cg + c] = s[c];
  }
  __syncthreads();
  if (t < D) {
    double acc = 0.0;
#pragma unroll
    for (int w = 0; w < kPackWaves; ++w) acc += red[w][t];
    S.partial[set][(bh * chunks + chunk) * D + t] = acc;
  }
}

// mu[bh][c] = float(sum over chunks / n).  One workgroup per (b, h): kThreads / D
// groups of threads take interleaved chunks and LDS adds the group sums (float64;
// the order of the additions moves mu by far less than one float32 ulp).
__global__ __launch_bounds__(kThreads) void mu_final_kernel(const Sets S, int64_t BH, int64_t n, int64_t chunks,
                                                            int D) {
  __shared__ double red[kThreads];
  const int set = (int)(blockIdx.x / BH);
  const int64_t bh = blockIdx.x % BH;
  const double* __restrict__ partial = S.partial[set];
  const int groups = kThreads / D;
  const int c = threadIdx.x % D, grp = threadIdx.x / D;
  double s = 0.0;
  for (int64_t k = grp; k < chunks; k += groups) s += partial[(bh * chunks + k) * D + c];
  red[threadIdx.x] = s;
  __syncthreads();
  if (grp == 0) {
    for (int q = 1; q < groups; ++q) s += red[q * D + c];
    S.mu[set][bh * D + c] = (float)(s / (double)n);
  }
}

// 32 channels (one code word) per lane, D/32 lanes per token row: the word
// needs no lane exchange, and a wave reads 64 consecutive 32-channel runs.
// MEAN_SIGN subtracts mu and sums |x - mu| in float64 for alpha (the D/32 lanes
// of a row add their partial sums).  Plain SIGN also writes mu = 0 when asked
// (mu_count = BH*D floats), so no separate fill launch is needed.
// FUSED (MEAN_SIGN, a workgroup's rows within at most two heads): mu is finished
// here instead of by mu_final_kernel, the first 2D threads summing the column
// partials of those heads into LDS; the workgroup holding a head's first row
// writes it.
template <typename T, int D, bool MEAN, bool FUSED>
__global__ __launch_bounds__(kThreads) void pack_rows_kernel(const Sets S, uint32_t rows, uint32_t n,
                                                             uint32_t per, uint32_t mu_count, uint32_t chunks) {
  constexpr int LPR = D / 32;
  constexpr int RPW = kThreads / LPR;  // rows per workgroup
  const int set = (int)(blockIdx.x / per);
  const uint32_t blk = blockIdx.x % per;
  const T* __restrict__ x = static_cast<const T*>(S.x[set]);
  const uint32_t tid = blk * kThreads + threadIdx.x;
  if (!MEAN && S.mu[set] != nullptr && tid < mu_count) S.mu[set][tid] = 0.0f;
  __shared__ float mus[FUSED ? 2 : 1][FUSED ? D : 1];
  const uint32_t h0 = blk * RPW / n;
  if (FUSED) {
    if (threadIdx.x < 2 * D) {
      const uint32_t hh = h0 + threadIdx.x / D, c = threadIdx.x % D;
      float m = 0.0f;
      if (hh < rows / n) {
        double acc = 0.0;
        for (uint32_t k = 0; k < chunks; ++k) acc += S.partial[set][((size_t)hh * chunks + k) * D + c];
        m = (float)(acc / (double)n);
        if ((size_t)hh * n >= (size_t)blk * RPW && (size_t)hh * n < (size_t)blk * RPW + RPW)
          S.mu[set][(size_t)hh * D + c] = m;
      }
      mus[threadIdx.x / D][c] = m;
    }
    __syncthreads();
  }
  const uint32_t r = tid / LPR, part = tid % LPR;
  const bool live = r < rows;
  const uint32_t rr = live ? r : rows - 1;  // dead lanes read a valid row, write nothing
  float v[32];
  const T* src = x + (size_t)rr * D + 32 * part;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float e[8];
    load8<T>(src + 8 * k, e);
#pragma unroll
    for (int c = 0; c < 8; ++c) v[8 * k + c] = e[c];
  }
  double asum = 0.0;
  if (MEAN) {
    const float* m = FUSED ? &mus[min(rr / n - h0, 1u)][32 * part] : S.mu[set] + (size_t)(rr / n) * D + 32 * part;
#pragma unroll
    for (int c = 0; c < 32; ++c) v[c] = __fsub_rn(v[c], m[c]);
#pragma unroll
    for (int c = 0; c < 32; ++c) asum += fabs((double)v[c]);
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) asum += __shfl_xor(asum, off, 64);
  }
  uint32_t w = 0;
#pragma unroll
  for (int c = 0; c < 32; ++c) w |= (uint32_t)(v[c] < 0.0f) << c;
  if (!live) return;
  S.bits[set][(size_t)r * (D / 32) + part] = w;
  if (part == 0 && S.alpha[set] != nullptr) S.alpha[set][r] = MEAN ? (float)(asum / (double)D) : 1.0f;
}

// MEAN_SIGN for heads of one column-sum chunk (n <= kPackChunk): one workgroup per
// (tensor, head) reads the head's rows into LDS once, then takes the column sums in the
// thread layout and order of colsum_partial_kernel, finishes mu as the row pass does,
// and runs the row pass of pack_rows_kernel from LDS (same lanes, same order), so the
// codes, alpha and mu are the same bits as the two-pass route with half the HBM reads.
template <typename T, int D>
// (five waves per SIMD: the head and the column sums take 27.5 KB of LDS at d = 64, so
// five workgroups fit a CU once the registers allow it)
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5)))
void pack_head_kernel(const Sets S, uint32_t BH, uint32_t n) {
  constexpr int TPR = D / 8;           // column pass: threads per token row
  constexpr int RPP = kThreads / TPR;  // rows per pass
  constexpr int LPR = D / 32;          // row pass: lanes per token row
  constexpr int RPW = kThreads / LPR;  // rows per pass
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t xbytes = (n * D * (uint32_t)sizeof(T) + 15u) & ~15u;
  T* xs = reinterpret_cast<T*>(smem);                             // [n][D]
  double* red = reinterpret_cast<double*>(smem + xbytes);         // [kPackWaves][D]
  float* mus = reinterpret_cast<float*>(red + kPackWaves * D);    // [D]
  const int set = (int)(blockIdx.x / BH);
  const size_t bh = blockIdx.x % BH;
  const int tid = threadIdx.x;
  {
    const uint8_t* src = static_cast<const uint8_t*>(S.x[set]) + bh * n * D * sizeof(T);
    const uint32_t total = n * D * (uint32_t)sizeof(T);  // a multiple of 16 (D * sizeof(T) >= 64)
    // eight 16-byte loads per thread in flight before their stores
    constexpr uint32_t kStep = kThreads * 16u;
    for (uint32_t base = (uint32_t)tid * 16u; base < total; base += 8u * kStep) {
      uint4 w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t o = base + k * kStep;
        w[k] = o < total ? *reinterpret_cast<const uint4*>(src + o) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t o = base + k * kStep;
        if (o < total) *reinterpret_cast<uint4*>(smem + o) = w[k];
      }
    }
  }
  __syncthreads();
  {
    const int r_off = tid / TPR, cg = tid % TPR;
    double sm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < kPackChunk / RPP; ++k) {
      const uint32_t r = (uint32_t)(r_off + RPP * k);
      if (r < n) {
        float v[8];
        load8<T>(xs + (size_t)r * D + 8 * cg, v);
#pragma unroll
        for (int c = 0; c < 8; ++c) sm[c] += (double)v[c];
      }
    }
    wave_colsum<D>(sm);
    if (tid % 64 < TPR) {
#pragma unroll
      for (int c = 0; c < 8; ++c) red[(tid / 64) * D + 8 * cg + c] = sm[c];
    }
  }
  __syncthreads();
  if (tid < D) {
    double part = 0.0;  // the chunk's partial, as colsum_partial_kernel forms it
#pragma unroll
    for (int w = 0; w < kPackWaves; ++w) part += red[w * D + tid];
    double acc = 0.0;  // the sum over the (one) chunk, as the row pass finishes it
    acc += part;
    const float m = (float)(acc / (double)n);
    mus[tid] = m;
    S.mu[set][bh * D + tid] = m;
  }
  __syncthreads();
  for (uint32_t r0 = 0; r0 < n; r0 += RPW) {
    const uint32_t r = r0 + (uint32_t)tid / LPR, part = (uint32_t)tid % LPR;
    const bool live = r < n;
    const uint32_t rr = live ? r : n - 1;
    float v[32];
    const T* src = xs + (size_t)rr * D + 32 * part;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float e[8];
      load8<T>(src + 8 * k, e);
#pragma unroll
      for (int c = 0; c < 8; ++c) v[8 * k + c] = e[c];
    }
    double asum = 0.0;
#pragma unroll
    for (int c = 0; c < 32; ++c) v[c] = __fsub_rn(v[c], mus[32 * part + c]);
#pragma unroll
    for (int c = 0; c < 32; ++c) asum += fabs((double)v[c]);
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) asum += __shfl_xor(asum, off, 64);
    uint32_t w = 0;
#pragma unroll
    for (int c = 0; c < 32; ++c) w |= (uint32_t)(v[c] < 0.0f) << c;
    if (live) {
      const size_t row = bh * n + r;
      S.bits[set][row * (D / 32) + part] = w;
      if (part == 0) S.alpha[set][row] = (float)(asum / (double)D);
    }
  }
}

// LDS bytes of pack_head_kernel for n tokens
template <typename T, int D>
uint32_t pack_head_lds(int64_t n) {
  return (uint32_t)(((n * D * (int64_t)sizeof(T) + 15) & ~(int64_t)15) + (int64_t)kPackWaves * D * 8 + D * 4);
}

template <typename T, int D>
hipError_t launch_typed(const PackParams& p, hipStream_t s) {
  Sets S{};
  for (int k = 0; k < p.count; ++k) {
    S.x[k] = p.set[k].x;
    S.bits[k] = p.set[k].bits;
    S.alpha[k] = p.set[k].alpha;
    S.mu[k] = p.set[k].mu;
    S.partial[k] = p.set[k].partial;
  }
  const unsigned cnt = (unsigned)p.count;
  const int64_t rows = p.BH * p.n;
  const int64_t threads = rows * (D / 32);
  if (p.mode == HAD_MEAN_SIGN && p.n <= kPackChunk) {
    // one chunk per head: one pass over x, from LDS
    const uint32_t lds = pack_head_lds<T, D>(p.n);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&pack_head_kernel<T, D>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)pack_head_lds<T, D>(kPackChunk));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((pack_head_kernel<T, D>), dim3(cnt * (unsigned)p.BH), dim3(kThreads), lds, s, S,
                       (uint32_t)p.BH, (uint32_t)p.n);
    return hipGetLastError();
  }
  if (p.mode == HAD_MEAN_SIGN) {
    const unsigned per = (unsigned)((threads + kThreads - 1) / kThreads);
    const int64_t chunks = pack_chunks(p.n);
    hipLaunchKernelGGL((colsum_partial_kernel<T, D>), dim3(cnt * (unsigned)(p.BH * chunks)), dim3(kThreads), 0,
                       s, S, p.n, chunks, p.BH * chunks);
    // a workgroup's rows span at most two heads, and re-summing their few partials per
    // workgroup costs less than a launch
    if (p.n >= kThreads / (D / 32) && chunks <= 4) {
      hipLaunchKernelGGL((pack_rows_kernel<T, D, true, true>), dim3(cnt * per), dim3(kThreads), 0, s, S,
                         (uint32_t)rows, (uint32_t)p.n, per, 0u, (uint32_t)chunks);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(mu_final_kernel, dim3(cnt * (unsigned)p.BH), dim3(kThreads), 0, s, S, p.BH, p.n, chunks, D);
    hipLaunchKernelGGL((pack_rows_kernel<T, D, true, false>), dim3(cnt * per), dim3(kThreads), 0, s, S,
                       (uint32_t)rows, (uint32_t)p.n, per, 0u, 0u);
  } else {
    // the launch covers max(rows * D/32, BH * D) threads per tensor: the first BH * D also write mu = 0
    const int64_t mu_count = p.BH * D;
    const int64_t need = std::max<int64_t>(threads, mu_count);
    const unsigned per = (unsigned)((need + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((pack_rows_kernel<T, D, false, false>), dim3(cnt * per), dim3(kThreads), 0, s, S,
                       (uint32_t)rows, (uint32_t)p.n, per, (uint32_t)mu_count, 0u);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dim(const PackParams& p, hipStream_t s) {
  switch (p.d) {
    case 32: return launch_typed<T, 32>(p, s);
    case 64: return launch_typed<T, 64>(p, s);
    case 128: return launch_typed<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_pack(const PackParams& p, hipStream_t s) {
  return p.x_dtype == HAD_BF16 ? launch_dim<uint16_t>(p, s) : launch_dim<float>(p, s);
}

}  // namespace had
