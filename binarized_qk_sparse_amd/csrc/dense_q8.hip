// BinaryAttention forward with the integer A*V contraction on int8 matrix cores.
//
// BinaryAttention, section 2.3 (Softmax(QK^T/sqrt(d) + B) V, QK^T from the
// binarized codes of section 2.2) and section 2.4 (mixed quantization):
//   A_q = clamp(rint(255 p), 0, 255)              uint8, scale 1/255
//   O   = float(sum_j A_q[j] Vq[j][c]) * scale[c] / 255
//
// gfx950 has no unsigned-by-signed int8 MFMA, so the kernel feeds
// A' = A_q - 128 (int8) and adds 128 * sum_j Vq[j][c] back:
//   sum_j A_q Vq = sum_j A' Vq + 128 sum_j Vq.
// Exact in int32 (|sum| <= 255 * 127 * 256 for the n <= 256 this kernel takes).
//
// One wave per 32-query tile; v_mfma_i32_32x32x16_i8 with
//   A (32 queries x 16 keys):  lane l holds row l%32, keys 8*(l/32)+0..7
//   B (16 keys x 32 channels): lane l holds column l%32, keys 8*(l/32)+0..7
//   C (32 x 32 int32):         lane l, element r: row 8*(r/4)+4*(l/32)+r%4, column l%32.
// Each lane computes the logits of exactly the A elements it feeds (VALU XOR +
// v_bcnt on the codes, LDS-staged key codes), keeps them in VGPRs for the
// row max / row sum / quantize passes, and the matrix cores do the contraction
// over all keys against the int8 V tile staged (transposed) in LDS.
#include <float.h>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

constexpr int kD = 64;
constexpr int kWaves = 4;
typedef int v16i __attribute__((ext_vector_type(16)));

struct DenseKArgs {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const float* aq;
  const float* ak;
  const float* bias;
  const int8_t* vq;
  const float* vscale;
  float* out;
  int H, n, npad, wgs_per_head;
  float isd;
};

template <int NK>  // key steps of 16; npad = 16 * NK >= n
__global__ __launch_bounds__(256) void dense_q8_kernel(const DenseKArgs a) {
  constexpr int NPAD = 16 * NK;
  __shared__ __align__(16) int8_t vqt[kD][NPAD];  // Vq transposed: [channel][key]
  __shared__ __align__(16) uint2 kcode[NPAD];
  __shared__ float akk[NPAD];
  __shared__ int colsum[kD];
  extern __shared__ float biasw[];  // [2n - 1]

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / a.wgs_per_head;
  const int part = blockIdx.x % a.wgs_per_head;
  const int hh = bh % a.H;
  const int n = a.n;

  // ---- stage codes, scales, bias table and the transposed int8 V of this head
  const uint2* kb = reinterpret_cast<const uint2*>(a.kbits) + (size_t)bh * n;
  for (int j = tid; j < NPAD; j += 256) {
    kcode[j] = j < n ? kb[j] : make_uint2(0u, 0u);
    akk[j] = (j < n && a.ak != nullptr) ? a.ak[(size_t)bh * n + j] : 1.0f;
  }
  if (a.bias != nullptr)
    for (int o = tid; o < 2 * n - 1; o += 256) biasw[o] = a.bias[(size_t)hh * (2 * n - 1) + o];
  const int8_t* vsrc = a.vq + (size_t)bh * n * kD;
  for (int e = tid; e < NPAD * kD; e += 256) {
    const int j = e / kD, c = e % kD;
    vqt[c][j] = j < n ? vsrc[(size_t)j * kD + c] : (int8_t)0;
  }
  __syncthreads();
  if (tid < kD) {
    int s = 0;
    for (int j = 0; j < NPAD; ++j) s += vqt[tid][j];
    colsum[tid] = s;
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int tile = part * kWaves + wave;
  if (tile * 32 >= n) return;
  const int r32 = lane & 31, khalf = lane >> 5;
  const int i = tile * 32 + r32;  // this lane's query row (may be padding)
  const int iq = i < n ? i : n - 1;
  const size_t row = (size_t)bh * n + iq;
  const uint2 qq = reinterpret_cast<const uint2*>(a.qbits)[row];
  const float aqv = a.aq != nullptr ? a.aq[row] : 1.0f;

  // ---- logits of this lane's A elements
  float lg[NK][8];
  float m = -INFINITY;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = ks * 16 + khalf * 8 + e;
      const uint2 kk = kcode[j];
      const int h = __builtin_popcount(qq.x ^ kk.x) + __builtin_popcount(qq.y ^ kk.y);
      const float b = (a.bias != nullptr && j < n) ? biasw[j - iq + n - 1] : 0.0f;
      float l = canonical_logit(aqv, akk[j], kD - 2 * h, a.isd, b);
      l = j < n ? l : -INFINITY;
      lg[ks][e] = l;
      m = fmaxf(m, l);
    }
  }
  m = fmaxf(m, __shfl_xor(m, 32, 64));  // the row's other 8-key half lives in lane ^ 32
  float z = 0.0f;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ex = __expf(lg[ks][e] - m);
      lg[ks][e] = ex;
      z += ex;
    }
  z += __shfl_xor(z, 32, 64);
  const float inv_z = 1.0f / z;

  // ---- quantize A and contract on the matrix cores
  v16i acc0 = {0}, acc1 = {0};
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qv = fminf(fmaxf(rintf(255.0f * (lg[ks][e] * inv_z)), 0.0f), 255.0f);
      const uint32_t a8 = (uint32_t)((int)qv - 128) & 0xffu;
      w[e >> 2] |= a8 << (8 * (e & 3));
    }
    const long A = (long)(((uint64_t)w[1] << 32) | w[0]);
    const long B0 = *reinterpret_cast<const long*>(&vqt[r32][ks * 16 + khalf * 8]);
    const long B1 = *reinterpret_cast<const long*>(&vqt[32 + r32][ks * 16 + khalf * 8]);
    acc0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(A, B0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(A, B1, acc1, 0, 0, 0);
  }

  // ---- dequantize and store
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int orow = tile * 32 + 8 * (r / 4) + 4 * khalf + (r % 4);
    if (orow < n) {
      float* o = a.out + ((size_t)bh * n + orow) * kD;
      const int c0 = r32, c1 = 32 + r32;
      const int t0 = acc0[r] + 128 * colsum[c0];
      const int t1 = acc1[r] + 128 * colsum[c1];
      o[c0] = __fdiv_rn(__fmul_rn((float)t0, a.vscale[(size_t)bh * kD + c0]), 255.0f);
      o[c1] = __fdiv_rn(__fmul_rn((float)t1, a.vscale[(size_t)bh * kD + c1]), 255.0f);
    }
  }
}

template <int NK>
hipError_t launch_nk(const DenseKArgs& ka, int64_t BH, hipStream_t s) {
  const dim3 grid((unsigned)(BH * ka.wgs_per_head));
  const size_t lds = ka.bias != nullptr ? sizeof(float) * (2 * ka.n - 1) : 0;
  hipLaunchKernelGGL((dense_q8_kernel<NK>), grid, dim3(256), lds, s, ka);
  return hipGetLastError();
}

}  // namespace

// Largest n the register-resident dense kernel takes.
int64_t dense_q8_max_n() { return 256; }

hipError_t launch_dense_q8(const AttnParams& p, hipStream_t s) {
  if (p.d != kD || p.n > dense_q8_max_n()) return hipErrorInvalidValue;
  DenseKArgs ka{};
  ka.qbits = p.qbits;
  ka.kbits = p.kbits;
  ka.aq = p.alpha_q;
  ka.ak = p.alpha_k;
  ka.bias = p.bias;
  ka.vq = static_cast<const int8_t*>(p.v);
  ka.vscale = p.vscale;
  ka.out = p.out;
  ka.H = (int)p.H;
  ka.n = (int)p.n;
  const int nk = (int)((p.n + 15) / 16);
  ka.npad = 16 * nk;
  const int tiles = (int)((p.n + 31) / 32);
  ka.wgs_per_head = (tiles + kWaves - 1) / kWaves;
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  const int64_t BH = p.B * p.H;
  if (nk <= 2) return launch_nk<2>(ka, BH, s);
  if (nk <= 4) return launch_nk<4>(ka, BH, s);
  if (nk <= 8) return launch_nk<8>(ka, BH, s);
  if (nk <= 13) return launch_nk<13>(ka, BH, s);
  return launch_nk<16>(ka, BH, s);
}

}  // namespace had
