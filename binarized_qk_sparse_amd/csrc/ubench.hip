// Measured ceilings of the units that bound the attention kernels, for the
// roofline next to the datasheet peaks: a chain of XOR + popcount (the integer
// VALU work of the Hamming logits, two lane-ops per step) and v_exp_f32 (the
// softmax exponential).  Measurement only: the attention path does not use this
// library.
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

}  // namespace

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
