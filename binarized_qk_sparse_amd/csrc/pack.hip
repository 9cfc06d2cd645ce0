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

// Column sums over one chunk of tokens, in float64: partial[bh][chunk][c].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void colsum_partial_kernel(const T* __restrict__ x, int64_t n,
                                                                  int64_t chunks,
                                                                  double* __restrict__ partial) {
  constexpr int TPR = D / 8;          // threads per token row
  constexpr int RPP = kThreads / TPR;  // rows per pass
  __shared__ double red[RPP][D];
  const int64_t bh = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x % chunks;
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
#pragma unroll
  for (int c = 0; c < 8; ++c) red[r_off][8 * cg + c] = s[c];
  __syncthreads();
  if (t < D) {
    double acc = 0.0;
    for (int rp = 0; rp < RPP; ++rp) acc += red[rp][t];
    partial[(bh * chunks + chunk) * D + t] = acc;
  }
}

// mu[bh][c] = float(sum over chunks / n).
__global__ __launch_bounds__(kThreads) void mu_final_kernel(const double* __restrict__ partial,
                                                            int64_t BH, int64_t n, int64_t chunks,
                                                            int D, float* __restrict__ mu) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= BH * D) return;
  const int64_t bh = id / D, c = id % D;
  double s = 0.0;
  for (int64_t k = 0; k < chunks; ++k) s += partial[(bh * chunks + k) * D + c];
  mu[id] = (float)(s / (double)n);
}

// One token row per D/8 lanes: code bits, and alpha for MEAN_SIGN.
template <typename T, int D, bool MEAN>
__global__ __launch_bounds__(kThreads) void pack_rows_kernel(const T* __restrict__ x, int64_t rows,
                                                             int64_t n, const float* __restrict__ mu,
                                                             uint32_t* __restrict__ bits,
                                                             float* __restrict__ alpha) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  constexpr int W = D / 32;
  const int t = threadIdx.x;
  const int cg = t % TPR;
  const int64_t r = (int64_t)blockIdx.x * RPP + t / TPR;
  const bool live = r < rows;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) load8<T>(x + r * D + 8 * cg, v);
  if (MEAN && live) {
    const float* m = mu + (r / n) * D + 8 * cg;
    const float4 m0 = *reinterpret_cast<const float4*>(m);
    const float4 m1 = *reinterpret_cast<const float4*>(m + 4);
    v[0] = __fsub_rn(v[0], m0.x); v[1] = __fsub_rn(v[1], m0.y);
    v[2] = __fsub_rn(v[2], m0.z); v[3] = __fsub_rn(v[3], m0.w);
    v[4] = __fsub_rn(v[4], m1.x); v[5] = __fsub_rn(v[5], m1.y);
    v[6] = __fsub_rn(v[6], m1.z); v[7] = __fsub_rn(v[7], m1.w);
  }
  uint32_t b8 = 0;
  double asum = 0.0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    b8 |= (uint32_t)(v[c] < 0.0f) << c;
    if (MEAN) asum += fabs((double)v[c]);
  }
  // four lanes (32 channels) make one word
  uint32_t w = b8 << (8 * (cg & 3));
  w |= __shfl_xor(w, 1, 64);
  w |= __shfl_xor(w, 2, 64);
  if (MEAN) {
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) asum += __shfl_xor(asum, off, 64);
  }
  if (!live) return;
  if ((cg & 3) == 0) bits[r * W + cg / 4] = w;
  if (cg == 0 && alpha != nullptr) alpha[r] = MEAN ? (float)(asum / (double)D) : 1.0f;
}

__global__ __launch_bounds__(kThreads) void fill_f32_kernel(float* __restrict__ p, int64_t count, float v) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < count) p[i] = v;
}

template <typename T, int D>
hipError_t launch_typed(const PackParams& p, hipStream_t s) {
  const T* x = static_cast<const T*>(p.x);
  const int64_t rows = p.BH * p.n;
  constexpr int RPP = kThreads / (D / 8);
  const unsigned grid = (unsigned)((rows + RPP - 1) / RPP);
  if (p.mode == HAD_MEAN_SIGN) {
    const int64_t chunks = pack_chunks(p.n);
    hipLaunchKernelGGL((colsum_partial_kernel<T, D>), dim3((unsigned)(p.BH * chunks)), dim3(kThreads), 0,
                       s, x, p.n, chunks, p.partial);
    const unsigned g2 = (unsigned)((p.BH * D + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(mu_final_kernel, dim3(g2), dim3(kThreads), 0, s, p.partial, p.BH, p.n, chunks, D,
                       p.mu);
    hipLaunchKernelGGL((pack_rows_kernel<T, D, true>), dim3(grid), dim3(kThreads), 0, s, x, rows, p.n,
                       p.mu, p.bits, p.alpha);
  } else {
    if (p.mu != nullptr) {
      const int64_t count = p.BH * D;
      hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((count + kThreads - 1) / kThreads)), dim3(kThreads),
                         0, s, p.mu, count, 0.0f);
    }
    hipLaunchKernelGGL((pack_rows_kernel<T, D, false>), dim3(grid), dim3(kThreads), 0, s, x, rows, p.n,
                       nullptr, p.bits, p.alpha);
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
