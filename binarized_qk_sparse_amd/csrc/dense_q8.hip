// BinaryAttention forward with the integer A*V contraction on int8 matrix cores.
//
// BinaryAttention, section 2.3 (Softmax(QK^T/sqrt(d) + B) V, QK^T from the
// binarized codes of section 2.2) and section 2.4 (mixed quantization):
//   A_q = clamp(rint(255 p), 0, 255)              uint8, scale 1/255
//   O   = float(sum_j A_q[j] Vq[j][c]) * scale[c] / 255
//
// gfx950 has no unsigned-by-signed int8 MFMA, so the kernel feeds
// A' = A_q - 128 (int8) and adds 128 * sum_j Vq[j][c] back:
//   sum_j A_q Vq = sum_j A' Vq + 128 sum_j Vq,
// exact in int32 (|sum| <= 255 * 127 * 256 for the n <= 256 this kernel takes).
//
// One wave per 16-query tile; v_mfma_i32_16x16x32_i8 with
//   A (16 queries x 32 keys):  lane l holds row l%16, keys 8*(l/16)+0..7
//   B (32 keys x 16 channels): lane l holds column l%16, keys 8*(l/16)+0..7
//   C (16 x 16 int32):         lane l, element r: row 4*(l/16)+r, column l%16.
// Each lane computes the logits of exactly the A elements it feeds (VALU XOR +
// v_bcnt on LDS-staged key codes), keeps them in VGPRs through the row max,
// row sum and quantize passes, and the matrix cores contract the quantized
// A against the transposed int8 V tile staged in LDS.
#include <float.h>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

// head_dim D is 64 or 128 (codes of D / 32 words, D / 16 channel tiles)
constexpr int kWaves = 4;
typedef int v4i __attribute__((ext_vector_type(4)));

struct DenseKArgs {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const float* aq;
  const float* ak;
  const float* bias;
  const int8_t* vq;
  const float* vscale;
  float* out;
  int H, n;
  float isd;
};

// Sum / max of a row whose values live in lanes l, l^16, l^32, l^48.
HAD_DEVICE float row4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
HAD_DEVICE float row4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

template <int NK, bool BIAS, int D>  // key steps of 32; NPAD = 32 * NK >= n
__global__ __launch_bounds__(256) void dense_q8_kernel(const DenseKArgs a) {
  constexpr int NPAD = 32 * NK;
  constexpr int NT = D / 16;  // channel tiles
  __shared__ __align__(16) int8_t vqt[D][NPAD];  // Vq transposed: [channel][key]
  __shared__ __align__(16) Code<D> kcode[NPAD];
  __shared__ __align__(16) float akk[NPAD];
  __shared__ int colsum[D];
  extern __shared__ float biasw[];  // [2n - 1 + NPAD]: the table, then zeros read by padding keys

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int hh = bh % a.H;
  const int n = a.n;

  // ---- stage codes, scales, bias table and the transposed int8 V of this head
  for (int j = tid; j < NPAD; j += 256) {
    Code<D> c = load_code<D>(a.kbits, (size_t)bh * n + (j < n ? j : 0));
    if (j >= n)
#pragma unroll
      for (int w = 0; w < D / 32; ++w) c.w[w] = 0u;
    kcode[j] = c;
    akk[j] = (j < n && a.ak != nullptr) ? a.ak[(size_t)bh * n + j] : 1.0f;
  }
  if (BIAS)
    for (int o = tid; o < 2 * n - 1 + NPAD; o += 256)
      biasw[o] = o < 2 * n - 1 ? a.bias[(size_t)hh * (2 * n - 1) + o] : 0.0f;
  // int8 V transposed, four keys x four channels per step: one 32-bit load per
  // key, a byte transpose by v_perm, one 32-bit LDS store per channel.  Threads
  // with consecutive ids take consecutive key blocks of one channel group, so the
  // stores of a wave fill consecutive words of the same rows.
  const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(a.vq + (size_t)bh * n * D);
  constexpr int KB = NPAD / 4;  // key blocks
  for (int e = tid; e < KB * (D / 4); e += 256) {
    const int jb = 4 * (e % KB), c4 = 4 * (e / KB);
    uint32_t w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      w[r] = jb + r < n ? *reinterpret_cast<const uint32_t*>(vsrc + (size_t)(jb + r) * D + c4) : 0u;
    const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
    const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
    const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 0][jb]) = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 1][jb]) = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 2][jb]) = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 3][jb]) = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
  }
  __syncthreads();
  // column sums of int8 V: four threads per channel, each a quarter of the key
  // blocks summed four keys at a time by v_dot4_i32_i8 against ones
  for (int e = tid; e < 4 * D; e += 256) {
    const int c = e >> 2, part = e & 3;
    int s = 0;
    for (int b = part; b < KB; b += 4)
      s = __builtin_amdgcn_sdot4(*reinterpret_cast<const int*>(&vqt[c][4 * b]), 0x01010101, s, false);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (part == 0) colsum[c] = s;
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int tiles = (n + 15) / 16;
  const float log2e = 1.4426950408889634f;
  for (int tile = wave; tile < tiles; tile += kWaves) {
    const int i = tile * 16 + r16;  // this lane's query row (may be padding)
    const int iq = i < n ? i : n - 1;
    const size_t row = (size_t)bh * n + iq;
    const Code<D> qq = load_code<D>(a.qbits, row);
    const float aqv = a.aq != nullptr ? a.aq[row] : 1.0f;
    const float* brow = biasw + (n - 1 - iq);  // bias of key j is brow[j]

    // ---- logits of this lane's A elements
    float lg[NK][8];
    float m = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int j0 = ks * 32 + kg * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        const int h = hamming<D>(qq, kcode[j]);
        const float b = BIAS ? brow[j] : 0.0f;
        float l = canonical_logit(aqv, akk[j], D - 2 * h, a.isd, b);
        if (ks == NK - 1) l = j < n ? l : -INFINITY;  // only the last step holds padding keys
        lg[ks][e] = l;
        m = fmaxf(m, l);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep each step's operand loads short-lived
    }
    m = row4_max(m);
    const float mb = m * log2e;
    float z = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ex = exp2f(__builtin_fmaf(lg[ks][e], log2e, -mb));
        lg[ks][e] = ex;
        z += ex;
      }
    const float q255 = 255.0f / row4_sum(z);

    // ---- quantize A and contract on the matrix cores
    v4i acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      // v_cvt_pk_u8_f32 rounds to nearest even, clamps to [0, 255] and writes
      // the byte in place: A_q four to a register; xor 0x80 turns each into A_q - 128
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(lg[ks][e] * q255, e & 3, w[e >> 2]);
      const long A = (long)((((uint64_t)w[1] << 32) | w[0]) ^ 0x8080808080808080ull);
      const int kk0 = ks * 32 + kg * 8;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const long B = *reinterpret_cast<const long*>(&vqt[nt * 16 + r16][kk0]);
        acc[nt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, acc[nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- dequantize and store
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int c = nt * 16 + r16;
      const float sc = a.vscale[(size_t)bh * D + c];
      const int cs = 128 * colsum[c];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int orow = tile * 16 + 4 * kg + r;
        if (orow < n)
          a.out[((size_t)bh * n + orow) * D + c] = __fdiv_rn(__fmul_rn((float)(acc[nt][r] + cs), sc), 255.0f);
      }
    }
  }
}

template <int NK, int D>
hipError_t launch_nkd(const DenseKArgs& ka, int64_t BH, hipStream_t s) {
  if (ka.bias != nullptr) {
    const size_t lds = sizeof(float) * (2 * ka.n - 1 + 32 * NK);
    hipLaunchKernelGGL((dense_q8_kernel<NK, true, D>), dim3((unsigned)BH), dim3(64 * kWaves), lds, s, ka);
  } else {
    hipLaunchKernelGGL((dense_q8_kernel<NK, false, D>), dim3((unsigned)BH), dim3(64 * kWaves), 0, s, ka);
  }
  return hipGetLastError();
}

template <int NK>
hipError_t launch_nk(const DenseKArgs& ka, int d, int64_t BH, hipStream_t s) {
  return d == 128 ? launch_nkd<NK, 128>(ka, BH, s) : launch_nkd<NK, 64>(ka, BH, s);
}

}  // namespace

// Largest n the register-resident dense kernel takes.
int64_t dense_q8_max_n() { return 256; }

hipError_t launch_dense_q8(const AttnParams& p, hipStream_t s) {
  if ((p.d != 64 && p.d != 128) || p.n > dense_q8_max_n()) return hipErrorInvalidValue;
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
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  const int nk = (int)((p.n + 31) / 32);
  const int64_t BH = p.B * p.H;
  switch (nk) {
    case 1: return launch_nk<1>(ka, (int)p.d, BH, s);
    case 2: return launch_nk<2>(ka, (int)p.d, BH, s);
    case 3: return launch_nk<3>(ka, (int)p.d, BH, s);
    case 4: return launch_nk<4>(ka, (int)p.d, BH, s);
    case 5: return launch_nk<5>(ka, (int)p.d, BH, s);
    case 6: return launch_nk<6>(ka, (int)p.d, BH, s);
    case 7: return launch_nk<7>(ka, (int)p.d, BH, s);
    default: return launch_nk<8>(ka, (int)p.d, BH, s);
  }
}

}  // namespace had
