// Measured ceilings of the units that bound the attention kernels, for the
// roofline next to the datasheet peaks: a chain of XOR + popcount (the integer
// VALU work of the Hamming logits, two lane-ops per step) and v_exp_f32 (the
// softmax exponential), and the VALU issue time a matrix-core product takes from
// the other work of its SIMD.  Measurement only: the attention path does not use
// this library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;  // independent chains per lane, so every issue slot can be filled

__global__ __launch_bounds__(kThreads) void xor_bcnt_kernel(uint32_t* out, int iters, uint32_t key) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  uint32_t a[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) a[k] = t * (2654435761u + 2u * k);
#pragma unroll 4
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) a[k] = (uint32_t)__builtin_popcount(a[k] ^ key) + a[k];  // v_xor, v_bcnt
  }
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s ^= a[k];
  out[t] = s;
}

__global__ __launch_bounds__(kThreads) void exp_kernel(float* out, int iters) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  float a[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) a[k] = (float)((t + k) & 255) * (1.0f / 256.0f);
#pragma unroll 4
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) a[k] = __builtin_amdgcn_exp2f(-a[k]);  // stays in (0, 1]
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += a[k];
  out[t] = s;
}

// 120 VALU instructions per iteration (40 steps of eight independent add / xor-add /
// popcount chains) and, with MFMA, ten independent v_mfma_f32_16x16x32_bf16 beside
// them.  Their difference in time, per product, is the VALU issue time a product takes.
template <bool MFMA>
__global__ __launch_bounds__(kThreads) void coissue_kernel(float* out, int iters, uint32_t seed) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  const int lane = (int)(threadIdx.x & 63u);
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)(lane + e);
    b[e] = (__bf16)(float)(lane - e);
  }
  f32x4 acc[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t x[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) x[k] = seed + t * kChains + k;
  for (int i = 0; i < iters; ++i) {
    if (MFMA) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int k = 0; k < 5; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 5; ++v)
#pragma unroll
      for (int k = 0; k < kChains; ++k) x[k] = (x[k] ^ (x[(k + 1) % kChains] + 0x9e3779b9u)) + __builtin_popcount(x[k]);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 5; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  uint32_t h = 0;
#pragma unroll
  for (int k = 0; k < kChains; ++k) h ^= x[k];
  out[t] = s + (float)h;
}

}  // namespace

// out: device buffer of blocks * 256 floats.  Per launch: blocks * 4 waves * iters *
// 120 VALU instructions, and as many times 10 matrix-core products when with_mfma.
extern "C" int hub_coissue(float* out, int blocks, int iters, int with_mfma, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return 1;
  if (with_mfma)
    hipLaunchKernelGGL(coissue_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out,
                       iters, 1u);
  else
    hipLaunchKernelGGL(coissue_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out,
                       iters, 1u);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// out: device buffer of blocks * 256 words.  Lane-ops per launch:
// blocks * 256 * iters * 8 chains * 2.
extern "C" int hub_xor_bcnt(uint32_t* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(xor_bcnt_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters,
                     0x9e3779b9u);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// out: device buffer of blocks * 256 floats.  v_exp_f32 per launch: blocks * 256 * iters * 8.
extern "C" int hub_exp(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(exp_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
