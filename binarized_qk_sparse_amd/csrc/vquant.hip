// Per-channel integer quantization of V (BinaryAttention, section 2.4: V is
// quantized per channel to int8 because its channels can hold outliers; the
// conclusion names 4-bit V as the next step), with L levels each side of zero,
// L = 127 (int8) or 7 (4-bit values):
//   scale[c] = max_j |V[j][c]| / L          (float32, correctly rounded)
//   Vq[j][c] = clamp(rint(V[j][c] / scale[c]), -L, L), 0 if scale is 0
// A streaming pass bound by HBM bandwidth: a max pass over V, then a quantize
// pass that reads V again and writes one byte per element (L = 127), or two
// 4-bit two's-complement codes per byte (L = 7): byte b of a row holds channel
// 2b in its low nibble and channel 2b + 1 in its high nibble.
#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

constexpr int kThreads = 256;

template <typename T>
HAD_DEVICE void load8v(const T* p, float (&v)[8]);
template <>
HAD_DEVICE void load8v<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
HAD_DEVICE void load8v<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
  v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
  v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void vmax_partial_kernel(const T* __restrict__ v, int64_t n,
                                                                int64_t chunks, float* __restrict__ partial) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  __shared__ float red[RPP][D];
  const int64_t bh = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x % chunks;
  const int t = threadIdx.x;
  const int r_off = t / TPR, cg = t % TPR;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t r0 = chunk * kVqChunk;
  for (int k = 0; k < kVqChunk / RPP; ++k) {
    const int64_t r = r0 + r_off + (int64_t)RPP * k;
    if (r < n) {
      float x[8];
      load8v<T>(v + (bh * n + r) * D + 8 * cg, x);
#pragma unroll
      for (int c = 0; c < 8; ++c) m[c] = fmaxf(m[c], fabsf(x[c]));
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) red[r_off][8 * cg + c] = m[c];
  __syncthreads();
  if (t < D) {
    float acc = 0.0f;
    for (int rp = 0; rp < RPP; ++rp) acc = fmaxf(acc, red[rp][t]);
    partial[(bh * chunks + chunk) * D + t] = acc;
  }
}

// scale[bh][c] = max over chunks / 127.  One workgroup per (b, h): kThreads / D
// groups of threads take interleaved chunks, LDS takes the max of the groups.
__global__ __launch_bounds__(kThreads) void vscale_kernel(const float* __restrict__ partial, int64_t chunks, int D,
                                                          float levels, float* __restrict__ scale) {
  __shared__ float red[kThreads];
  const int64_t bh = blockIdx.x;
  const int groups = kThreads / D;
  const int c = threadIdx.x % D, grp = threadIdx.x / D;
  float m = 0.0f;
  for (int64_t k = grp; k < chunks; k += groups) m = fmaxf(m, partial[(bh * chunks + k) * D + c]);
  red[threadIdx.x] = m;
  __syncthreads();
  if (grp == 0) {
    for (int q = 1; q < groups; ++q) m = fmaxf(m, red[q * D + c]);
    scale[bh * D + c] = __fdiv_rn(m, levels);
  }
}

template <int D, int L>
HAD_DEVICE void store_codes(int8_t* __restrict__ vq, uint32_t r, int cg, const uint32_t (&b)[8]) {
  if constexpr (L == 7) {
    // eight 4-bit codes in one word: nibble c is channel 8 cg + c
    uint32_t o = 0u;
#pragma unroll
    for (int c = 0; c < 8; ++c) o |= (b[c] & 0xfu) << (4 * c);
    *reinterpret_cast<uint32_t*>(vq + (size_t)r * (D / 2) + 4 * cg) = o;
  } else {
    uint2 o;
    o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    *reinterpret_cast<uint2*>(vq + (size_t)r * D + 8 * cg) = o;
  }
}

template <typename T, int D, int L>
__global__ __launch_bounds__(kThreads) void vq_kernel(const T* __restrict__ v, uint32_t rows, uint32_t n,
                                                      const float* __restrict__ scale, int8_t* __restrict__ vq) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  const int t = threadIdx.x;
  const int cg = t % TPR;
  const uint32_t r = blockIdx.x * RPP + t / TPR;
  if (r >= rows) return;
  float x[8];
  load8v<T>(v + (size_t)r * D + 8 * cg, x);
  const float4* sp = reinterpret_cast<const float4*>(scale + (size_t)(r / n) * D + 8 * cg);
  const float4 s0 = sp[0], s1 = sp[1];
  const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  uint32_t b[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) b[c] = quant_i8<L>(x[c], s[c], __builtin_amdgcn_rcpf(s[c]));
  store_codes<D, L>(vq, r, cg, b);
}

// The quantize pass with the scales finished in the same launch: when a
// workgroup's rows span at most two (b, h) slices (n >= rows per workgroup), its
// first 2D threads take the max over the chunk partials of those slices and
// divide by L (as vscale_kernel does) into LDS; the workgroup holding a slice's
// first row writes its scales.
template <typename T, int D, int L>
__global__ __launch_bounds__(kThreads) void vq_fused_kernel(const T* __restrict__ v, uint32_t rows, uint32_t n,
                                                            uint32_t chunks, const float* __restrict__ partial,
                                                            float* __restrict__ scale, int8_t* __restrict__ vq) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  __shared__ float sc[2][D];
  const uint32_t r0 = blockIdx.x * RPP;
  const uint32_t h0 = r0 / n;
  const uint32_t nh = rows / n;
  if (threadIdx.x < 2 * D) {
    const uint32_t hh = h0 + threadIdx.x / D, c = threadIdx.x % D;
    float q = 0.0f;
    if (hh < nh) {
      float m = 0.0f;
      for (uint32_t k = 0; k < chunks; ++k) m = fmaxf(m, partial[((size_t)hh * chunks + k) * D + c]);
      q = __fdiv_rn(m, (float)L);
      if ((size_t)hh * n >= r0 && (size_t)hh * n < (size_t)r0 + RPP) scale[(size_t)hh * D + c] = q;
    }
    sc[threadIdx.x / D][c] = q;
  }
  __syncthreads();
  const int t = threadIdx.x;
  const int cg = t % TPR;
  const uint32_t r = r0 + t / TPR;
  if (r >= rows) return;
  float x[8];
  load8v<T>(v + (size_t)r * D + 8 * cg, x);
  const float* sp = &sc[min(r / n - h0, 1u)][8 * cg];
  uint32_t b[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) b[c] = quant_i8<L>(x[c], sp[c], __builtin_amdgcn_rcpf(sp[c]));
  store_codes<D, L>(vq, r, cg, b);
}

// Eight elements from the registers one 16-byte load (bf16) or two (fp32) filled.
template <typename T>
HAD_DEVICE void unpack8(const uint4 (&w)[sizeof(T) / 2], float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    x[0] = bf16_lo(w[0].x); x[1] = bf16_hi(w[0].x);
    x[2] = bf16_lo(w[0].y); x[3] = bf16_hi(w[0].y);
    x[4] = bf16_lo(w[0].z); x[5] = bf16_hi(w[0].z);
    x[6] = bf16_lo(w[0].w); x[7] = bf16_hi(w[0].w);
  } else {
    const uint32_t u[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = __builtin_bit_cast(float, u[c]);
  }
}

// Heads of at most kVqChunk rows in one launch: one workgroup per (b, h) loads the
// head's rows into registers (rows r_off + RPP k, eight channels per thread), takes
// the channel maxima of |V| (per thread, then a butterfly over the lanes of a wave
// that hold the same channels, then the waves through LDS), divides them by L as
// vscale_kernel does, and quantizes the rows it holds.  V is read once instead of
// twice, with the same bits: a maximum does not depend on the order it is taken in.
template <typename T, int D, int L>
__global__ __launch_bounds__(kThreads) void vq_head_kernel(const T* __restrict__ v, uint32_t n,
                                                           float* __restrict__ scale, int8_t* __restrict__ vq) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  constexpr int PASSES = kVqChunk / RPP;
  constexpr int NW = sizeof(T) / 2;  // 16-byte words per eight elements
  __shared__ float red[kThreads / 64][D];
  __shared__ float sc[D];
  const size_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const int r_off = t / TPR, cg = t % TPR;
  const uint4* src = reinterpret_cast<const uint4*>(v + bh * n * D);
  uint4 raw[PASSES][NW];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const uint32_t r = (uint32_t)(r_off + RPP * k);
#pragma unroll
    for (int w = 0; w < NW; ++w)
      raw[k][w] = r < n ? src[((size_t)r * D + 8 * cg) / (8 / NW) + w] : make_uint4(0u, 0u, 0u, 0u);
  }
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    float x[8];
    unpack8<T>(raw[k], x);
#pragma unroll
    for (int c = 0; c < 8; ++c) m[c] = fmaxf(m[c], fabsf(x[c]));  // (rows past n hold zeros)
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) m[c] = butterfly_f32<TPR>(m[c], [](float a, float b) { return fmaxf(a, b); });
  if (t % 64 < TPR) {
#pragma unroll
    for (int c = 0; c < 8; ++c) red[t / 64][8 * cg + c] = m[c];
  }
  __syncthreads();
  if (t < D) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) acc = fmaxf(acc, red[w][t]);
    const float q = __fdiv_rn(acc, (float)L);
    sc[t] = q;
    scale[bh * D + t] = q;
  }
  __syncthreads();
  float sv[8], inv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    sv[c] = sc[8 * cg + c];
    inv[c] = __builtin_amdgcn_rcpf(sv[c]);
  }
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const uint32_t r = (uint32_t)(r_off + RPP * k);
    if (r < n) {
      float x[8];
      unpack8<T>(raw[k], x);
      uint32_t b[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) b[c] = quant_i8<L>(x[c], sv[c], inv[c]);
      store_codes<D, L>(vq, (uint32_t)(bh * n) + r, cg, b);
    }
  }
}

template <typename T, int D, int L>
hipError_t launch_levels(const VQuantParams& p, hipStream_t s) {
  const T* v = static_cast<const T*>(p.v);
  if (p.n <= kVqChunk) {
    hipLaunchKernelGGL((vq_head_kernel<T, D, L>), dim3((unsigned)p.BH), dim3(kThreads), 0, s, v, (uint32_t)p.n,
                       p.vscale, p.vq);
    return hipGetLastError();
  }
  const int64_t chunks = vq_chunks(p.n);
  hipLaunchKernelGGL((vmax_partial_kernel<T, D>), dim3((unsigned)(p.BH * chunks)), dim3(kThreads), 0, s, v,
                     p.n, chunks, p.vmax_partial);
  // a workgroup's rows span at most two slices, and taking the max of their few partials
  // per workgroup costs less than a launch
  if (p.n >= kThreads / (D / 8) && chunks <= 4) {
    const int64_t rows = p.BH * p.n;
    constexpr int RPP = kThreads / (D / 8);
    hipLaunchKernelGGL((vq_fused_kernel<T, D, L>), dim3((unsigned)((rows + RPP - 1) / RPP)), dim3(kThreads), 0, s,
                       v, (uint32_t)rows, (uint32_t)p.n, (uint32_t)chunks, p.vmax_partial, p.vscale, p.vq);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(vscale_kernel, dim3((unsigned)p.BH), dim3(kThreads), 0, s, p.vmax_partial, chunks, D, (float)L,
                     p.vscale);
  const int64_t rows = p.BH * p.n;
  constexpr int RPP = kThreads / (D / 8);
  hipLaunchKernelGGL((vq_kernel<T, D, L>), dim3((unsigned)((rows + RPP - 1) / RPP)), dim3(kThreads), 0, s, v,
                     (uint32_t)rows, (uint32_t)p.n, p.vscale, p.vq);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const VQuantParams& p, hipStream_t s) {
  return p.levels == 7 ? launch_levels<T, D, 7>(p, s) : launch_levels<T, D, 127>(p, s);
}

template <typename T>
hipError_t launch_dim(const VQuantParams& p, hipStream_t s) {
  switch (p.d) {
    case 32: return launch_typed<T, 32>(p, s);
    case 64: return launch_typed<T, 64>(p, s);
    case 128: return launch_typed<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_vquant(const VQuantParams& p, hipStream_t s) {
  return p.v_dtype == HAD_BF16 ? launch_dim<uint16_t>(p, s) : launch_dim<float>(p, s);
}

}  // namespace had
