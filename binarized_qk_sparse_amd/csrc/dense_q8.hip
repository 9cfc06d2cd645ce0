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

#include <type_traits>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

// head_dim D is 64 or 128 (codes of D / 32 words, D / 16 channel tiles)
constexpr int kWaves = 4;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Bit b of a code byte to bit 3 of nibble b, 0x9 (-0.5) to 0x1 (+0.5) for a key (x = -1 at a
// set bit: -x/2 = +0.5), 0x2 (+1) to 0xA (-1) for a query: the fp4 (e2m1) operands of the
// distance products.
HAD_DEVICE uint32_t fp4_spread(uint32_t byte) {
  uint32_t sp = byte;
  sp = (sp | (sp << 12)) & 0x000f000fu;
  sp = (sp | (sp << 6)) & 0x03030303u;
  sp = (sp | (sp << 3)) & 0x11111111u;
  return sp << 3;
}

// Byte offset of the 16-byte half h (dims 32 h .. 32 h + 31) of key kk of a 32-key step
// among the step's fp4 key operands: the step's four 8-key blocks take 256 bytes each, a
// key's halves sit at slots 2 (kk % 8) + h, and block q flips slot bits 0 and 3 by q, so that
// the 16 lanes of one K-block (keys 8 q + e, e < 4, of the four blocks) read 16 different
// 16-byte slots.
HAD_DEVICE uint32_t fp4_key_offset(uint32_t kk, uint32_t h) {
  const uint32_t q = kk >> 3;
  const uint32_t slot = (2u * (kk & 7u) + h) ^ ((q & 1u) | ((q >> 1) << 3));
  return q * 256u + slot * 16u;
}

// The fp4 operands of one key (32 bytes at head_dim 64, 64 at 128) into the step's block.
template <int D>
HAD_DEVICE void store_fp4_key(uint8_t* kx, const Code<D>& c, uint32_t j);

// Word b (0..3) of a code by bitwise selects on masks the compiler cannot see through (a
// chain of selects on b is otherwise turned into a dynamic index, which puts the code in
// scratch memory).
template <int D>
HAD_DEVICE uint32_t code_word_sel(const Code<D>& c, uint32_t b) {
  if constexpr (D == 64) {
    uint32_t m = 0u - (b & 1u);
    asm volatile("" : "+v"(m));
    return (c.w[1] & m) | (c.w[0] & ~m);
  } else {
    uint32_t m1 = 0u - (b & 1u), m2 = 0u - ((b >> 1) & 1u);
    asm volatile("" : "+v"(m1), "+v"(m2));
    const uint32_t w01 = (c.w[1] & m1) | (c.w[0] & ~m1);
    const uint32_t w23 = (c.w[3] & m1) | (c.w[2] & ~m1);
    return (w23 & m2) | (w01 & ~m2);
  }
}

// Head_dim 128: byte offset of K-block b (dims 32 b .. 32 b + 31) of key kk of a step, 64
// bytes a key, the block index flipped by the key's lane group kk / 8 so that the 16 lanes
// of a K-block (four groups by four keys) read 16 different 16-byte slots.
HAD_DEVICE uint32_t fp4_key_offset128(uint32_t kk, uint32_t b) { return (kk * 4u + (b ^ ((kk >> 3) & 3u))) * 16u; }

template <int D>
HAD_DEVICE void store_fp4_key(uint8_t* kx, const Code<D>& c, uint32_t j) {
  const uint32_t ks = j >> 5, kk = j & 31u;
#pragma unroll
  for (int h = 0; h < D / 32; ++h) {
    const uint32_t w = c.w[h];
    const uint32_t off = D == 64 ? fp4_key_offset(kk, (uint32_t)h) : fp4_key_offset128(kk, (uint32_t)h);
    *reinterpret_cast<uint4*>(kx + ks * (32u * (D / 2)) + off) =
        make_uint4(0x99999999u ^ fp4_spread(w & 0xffu), 0x99999999u ^ fp4_spread((w >> 8) & 0xffu),
                   0x99999999u ^ fp4_spread((w >> 16) & 0xffu), 0x99999999u ^ fp4_spread(w >> 24));
  }
}

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
  // two-dimensional decomposable bias in place of `bias` (brow2 != NULL)
  const float* brow2;
  const float* bcol2;
  const float* bcls2;
  int gh, gw, cls;
  // fused entry point: raw Q, K, V (each fp32 or bf16) instead of the above
  const void* xq;
  const void* xk;
  const void* xv;
  int qk_bf16, v_bf16, mean;
};

// Eight consecutive elements from index i of a fp32 or bf16 tensor (16- or 32-byte read).
HAD_DEVICE void load8_any(const void* base, size_t i, bool bf16, float (&v)[8]) {
  if (bf16) {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
    v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
    v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Four consecutive elements (8- or 16-byte read).
HAD_DEVICE void load4_any(const void* base, size_t i, bool bf16, float (&v)[4]) {
  if (bf16) {
    const uint2 a = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
    v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
}

// Sum / max of a row whose values live in lanes l, l^16, l^32, l^48.
HAD_DEVICE float row4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
HAD_DEVICE float row4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// FUSED (binattn_dense_q8_fused): the workgroup also binarizes Q and K and
// quantizes V of its head into LDS first, with the arithmetic, thread layout
// and summation order of the separate passes (had_pack's column sums, codes and
// alpha; the V scale and int8 codes of the attention entry points), so both
// routes give the same bits.
// B2 (with BIAS): the two-dimensional bias, a separate instance so that the 1-D
// path carries none of its code.
template <int NK, bool BIAS, int D, bool FUSED, bool B2 = false>  // key steps of 32; NPAD = 32 * NK >= n
__global__ __launch_bounds__(256) void dense_q8_kernel(const DenseKArgs a) {
  constexpr int NPAD = 32 * NK;
  constexpr int NT = D / 16;  // channel tiles
  constexpr int FP = FUSED ? NPAD : 1;
  constexpr int FD = FUSED ? D : 1;
  constexpr int RPP = 256 / (D / 8);  // rows per pass with eight channels per thread
  __shared__ __align__(16) int8_t vqt[D][NPAD];  // Vq transposed: [channel][key]
  __shared__ __align__(16) Code<D> kcode[FUSED ? NPAD : 1];  // fused: the key codes, expanded after staging
  // the keys' fp4 operands of the distance products, 32 bytes a key at head_dim 64, 64 at 128
  // (fused: in the column-sum partials' space, which is dead by then)
  __shared__ __align__(256) uint8_t kx_own[FUSED ? 16 : NPAD * (D / 2)];
  __shared__ __align__(16) float akk[NPAD];
  __shared__ int colsum[D];
  __shared__ __align__(16) Code<D> qcode[FP];      // fused: query codes
  __shared__ float aqs[FP];                        // fused: query alphas
  __shared__ float vsc[FD];                        // fused: V scales
  __shared__ float mus[FUSED ? 2 : 1][FD];         // fused: mu of Q and K
  __shared__ __align__(256) double dred[FUSED ? RPP : 1][FD];  // fused: column-sum partials
  __shared__ float fred[FUSED ? RPP : 1][FD];      // fused: column-max partials
  // BIAS: the 1-D table [2n - 1 + NPAD] (zeros read by padding keys), or the
  // two-dimensional tables followed by the key position codes [NPAD]
  extern __shared__ float biasw[];
  static_assert(!FUSED || sizeof(dred) >= NPAD * (D / 2), "fp4 key operands fit the partials' space");
  uint8_t* const kx = FUSED ? reinterpret_cast<uint8_t*>(&dred[0][0]) : kx_own;

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int hh = bh % a.H;
  const int n = a.n;

  if constexpr (FUSED) {
    const bool qkb = a.qk_bf16 != 0, vb = a.v_bf16 != 0, mean = a.mean != 0;
    const int r_off = tid / (D / 8), cg = tid % (D / 8);
    // Column passes: thread (r_off, cg) takes channels 8 cg .. 8 cg + 7 of rows
    // r_off + RPP k, k ascending (the separate passes' layout and order); four
    // rows' reads are issued before any is used.
    auto col_pass = [&](const void* x, bool bf16, auto&& use) {
      constexpr int IT = 256 / RPP;  // rows per thread (n <= 256)
      constexpr int G = IT < 4 ? IT : 4;
#pragma unroll
      for (int k0 = 0; k0 < IT; k0 += G) {
        float v[G][8];
#pragma unroll
        for (int u = 0; u < G; ++u) {
          const int r = r_off + RPP * (k0 + u);
          if (r < n) load8_any(x, ((size_t)bh * n + r) * D + 8 * cg, bf16, v[u]);
        }
#pragma unroll
        for (int u = 0; u < G; ++u)
          if (r_off + RPP * (k0 + u) < n) use(v[u]);
      }
    };
    // ---- mu (mean reading): per-channel column sums in float64 over the head's tokens
    if (mean) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        double sm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        col_pass(t == 0 ? a.xq : a.xk, qkb, [&](const float(&v)[8]) {
#pragma unroll
          for (int c = 0; c < 8; ++c) sm[c] += (double)v[c];
        });
#pragma unroll
        for (int c = 0; c < 8; ++c) dred[r_off][8 * cg + c] = sm[c];
        __syncthreads();
        if (tid < D) {
          double acc = 0.0;
          for (int rp = 0; rp < RPP; ++rp) acc += dred[rp][tid];
          mus[t][tid] = (float)((0.0 + acc) / (double)n);
        }
        __syncthreads();
      }
    }
    // ---- V scales: per-channel max |v| over the head's tokens, / 127
    {
      float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      col_pass(a.xv, vb, [&](const float(&v)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) mx[c] = fmaxf(mx[c], fabsf(v[c]));
      });
#pragma unroll
      for (int c = 0; c < 8; ++c) fred[r_off][8 * cg + c] = mx[c];
    }
    // ---- codes (x - mu < 0, or x < 0) and alpha = mean |x - mu|: D/32 lanes per token
    constexpr int LPR = D / 32;
    constexpr int RPW = 256 / LPR;
    const int part = tid % LPR;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const void* x = t == 0 ? a.xq : a.xk;
      for (int r0 = 0; r0 < n; r0 += RPW) {
        const int r = r0 + tid / LPR;
        const bool live = r < n;
        const int rr = live ? r : n - 1;  // dead lanes read a valid row, write nothing
        float v[32];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float e[8];
          load8_any(x, ((size_t)bh * n + rr) * D + 32 * part + 8 * k, qkb, e);
#pragma unroll
          for (int c = 0; c < 8; ++c) v[8 * k + c] = e[c];
        }
        double asum = 0.0;
        if (mean) {
          const float* m = &mus[t][32 * part];
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
        if (live) {
          (t == 0 ? qcode : kcode)[rr].w[part] = w;
          if (part == 0) (t == 0 ? aqs : akk)[rr] = mean ? (float)(asum / (double)D) : 1.0f;
        }
      }
    }
    for (int j = n + tid; j < NPAD; j += 256) {  // padding keys: code 0, alpha 1
#pragma unroll
      for (int w = 0; w < D / 32; ++w) kcode[j].w[w] = 0u;
      akk[j] = 1.0f;
    }
    __syncthreads();  // the column maxima of V are in LDS
    if (tid < D) {
      float acc = 0.0f;
      for (int rp = 0; rp < RPP; ++rp) acc = fmaxf(acc, fred[rp][tid]);
      vsc[tid] = __fdiv_rn(acc, 127.0f);
    }
    __syncthreads();
  }

  // ---- stage codes, scales, bias table and the transposed int8 V of this head
  // (not fused: every global load of the staging below -- key codes and scales, the
  // bias window, int8 V -- is issued before the first store, one memory round trip)
  static_assert(NPAD <= 256, "one key per thread");
  Code<D> kc_st{};
  float ak_st = 1.0f;
  if constexpr (!FUSED) {
    const int j = tid;
    if (j < NPAD) {
      kc_st = load_code<D>(a.kbits, (size_t)bh * n + (j < n ? j : 0));
      ak_st = (j < n && a.ak != nullptr) ? a.ak[(size_t)bh * n + j] : 1.0f;
    }
  }
  constexpr bool b2 = BIAS && B2;
  uint32_t* kposs = reinterpret_cast<uint32_t*>(biasw + (b2 ? bias2d_floats(a.gh, a.gw, a.cls) : 0));
  constexpr int BIT = (3 * NPAD + 255) / 256;  // 1-D bias window floats per thread: 2n - 1 + NPAD <= 3 NPAD
  float bv[BIT];
  if (BIAS) {
    if (b2) {
      stage_bias2d(biasw, a.brow2, a.bcol2, a.bcls2, hh, a.gh, a.gw, a.cls, tid, 256);
      for (int j = tid; j < NPAD; j += 256) kposs[j] = bias2d_key(j < n ? j : n - 1, a.gh, a.gw, a.cls);
    } else {
#pragma unroll
      for (int u = 0; u < BIT; ++u) {
        const int o = tid + 256 * u;
        bv[u] = o < 2 * n - 1 ? a.bias[(size_t)hh * (2 * n - 1) + o] : 0.0f;
      }
    }
  }
  // int8 V transposed, four keys x four channels per step: one 32-bit load per
  // key, a byte transpose by v_perm, one 32-bit LDS store per channel.  Threads
  // with consecutive ids take consecutive key blocks of one channel group, so the
  // stores of a wave fill consecutive words of the same rows.
  // (fused: the int8 codes come from V itself, with the scales above)
  constexpr int KB = NPAD / 4;  // key blocks
  auto transpose_store = [&](int e, const uint32_t (&w)[4]) {
    const int jb = 4 * (e % KB), c4 = 4 * (e / KB);
    const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
    const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
    const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 0][jb]) = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 1][jb]) = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 2][jb]) = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    *reinterpret_cast<uint32_t*>(&vqt[c4 + 3][jb]) = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
  };
  if constexpr (!FUSED) {
    // every thread's loads of int8 V are in flight before the first is used (at most
    // NK / 2 items of four 32-bit loads each at head_dim 64)
    constexpr int VIT = (KB * (D / 4) + 255) / 256;
    const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(a.vq + (size_t)bh * n * D);
    uint32_t wv[VIT][4];
#pragma unroll
    for (int u = 0; u < VIT; ++u) {
      const int e = tid + 256 * u;
      const int jb = 4 * (e % KB), c4 = 4 * (e / KB);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        wv[u][r] = (e < KB * (D / 4) && jb + r < n) ? *reinterpret_cast<const uint32_t*>(vsrc + (size_t)(jb + r) * D + c4)
                                                    : 0u;
    }
#pragma unroll
    for (int u = 0; u < VIT; ++u)
      if (tid + 256 * u < KB * (D / 4)) transpose_store(tid + 256 * u, wv[u]);
  }
  if (BIAS && !b2) {
#pragma unroll
    for (int u = 0; u < BIT; ++u)
      if (tid + 256 * u < 2 * n - 1 + NPAD) biasw[tid + 256 * u] = bv[u];
  }
  if constexpr (!FUSED) {
    if (tid < NPAD) {
      if (tid >= n)
#pragma unroll
        for (int w = 0; w < D / 32; ++w) kc_st.w[w] = 0u;
      store_fp4_key<D>(kx, kc_st, (uint32_t)tid);
      akk[tid] = ak_st;
    }
  }
  if constexpr (FUSED) {
  for (int e = tid; e < KB * (D / 4); e += 256) {
    const int jb = 4 * (e % KB), c4 = 4 * (e / KB);
    uint32_t w[4];
    {
      float s4[4], inv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s4[c] = vsc[c4 + c];
        inv[c] = __builtin_amdgcn_rcpf(s4[c]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w[r] = 0u;
        if (jb + r < n) {
          float x[4];
          load4_any(a.xv, ((size_t)bh * n + jb + r) * D + c4, a.v_bf16 != 0, x);
#pragma unroll
          for (int c = 0; c < 4; ++c) w[r] |= quant_i8(x[c], s4[c], inv[c]) << (8 * c);
        }
      }
    }
    transpose_store(e, w);
  }
  }
  __syncthreads();
  if constexpr (FUSED) {
    // the keys' fp4 operands (one key per thread), now that the partials' space is free
    if (tid < NPAD) store_fp4_key<D>(kx, kcode[tid], (uint32_t)tid);
  }
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
    Code<D> qq;
    float aqv;
    if constexpr (FUSED) {
      qq = qcode[iq];
      aqv = aqs[iq];
    } else {
      qq = load_code<D>(a.qbits, row);
      aqv = a.aq != nullptr ? a.aq[row] : 1.0f;
    }
    const float* brow = biasw + (n - 1 - iq);  // 1-D table: bias of key j is brow[j]
    const int2 qb2 = b2 ? bias2d_query(iq, a.gh, a.gw, a.cls) : make_int2(0, 0);

    // ---- logits of this lane's A elements.  Head_dim 64: the distances of a 32-key step
    // from one fp4 product (as in the matrix-core top-N kernel): row 4 g + e of A holds key
    // 8 g + e in K-blocks 0, 1 and key 8 g + 4 + e in K-blocks 2, 3 (scaled by 2^8), column
    // r of B query r; from C = 2^22 + 32 + 256 * 32 the result is 2^22 + h0 + 256 h1
    // exactly, whose float bits hold 2 h0 in byte 0 and 2 h1 in byte 1: lane (g, r) gets
    // the eight distances of its A elements, d - 2h = 64 - byte.
    // Head_dim 128: K = 128 fills a product with one key block, so two products per step:
    // in product p row 4 g + e holds key 8 g + 4 p + e, K-block g' its dims 32 g' ..; from
    // C = 2^22 + 64 the result is 2^22 + h and d - 2h = 2^23 + 128 - 2C, exact in one fma.
    v8i Bq{};
    int scale_a = 127;
    {
      const uint32_t qw = code_word_sel<D>(qq, (uint32_t)(D == 64 ? (kg & 1) : kg));
#pragma unroll
      for (int b = 0; b < 4; ++b) Bq[b] = (int)(0x22222222u ^ fp4_spread((qw >> (8 * b)) & 0xffu));
      if constexpr (D == 64) scale_a = kg >= 2 ? 127 + 8 : 127;  // E8M0 2^8 for the second key block
    }
    uint32_t koff[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      koff[p] = D == 64 ? fp4_key_offset((uint32_t)(8 * (r16 >> 2) + (r16 & 3) + 4 * (kg >> 1)), (uint32_t)(kg & 1))
                        : fp4_key_offset128((uint32_t)(8 * (r16 >> 2) + 4 * p + (r16 & 3)), (uint32_t)kg);
    float lg[NK][8];
    float m = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int j0 = ks * 32 + kg * 8;
      float dotf[8];
      if constexpr (D == 128) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint4 av = *reinterpret_cast<const uint4*>(kx + ks * 2048 + koff[p]);
          v8i A{};
          A[0] = (int)av.x; A[1] = (int)av.y; A[2] = (int)av.z; A[3] = (int)av.w;
          constexpr float kC0 = 4194304.0f + 64.0f;
          f32x4 c = f32x4{kC0, kC0, kC0, kC0};
          c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bq, c, 4, 4, 0, 127, 0, 127);
          const float c0 = c[0], c1 = c[1], c2 = c[2], c3 = c[3];
          constexpr float kDot0 = 8388608.0f + 128.0f;  // 2^23 + 128
          dotf[4 * p + 0] = __builtin_fmaf(c0, -2.0f, kDot0);
          dotf[4 * p + 1] = __builtin_fmaf(c1, -2.0f, kDot0);
          dotf[4 * p + 2] = __builtin_fmaf(c2, -2.0f, kDot0);
          dotf[4 * p + 3] = __builtin_fmaf(c3, -2.0f, kDot0);
        }
      } else {
        const uint4 av = *reinterpret_cast<const uint4*>(kx + ks * 1024 + koff[0]);
        v8i A{};
        A[0] = (int)av.x; A[1] = (int)av.y; A[2] = (int)av.z; A[3] = (int)av.w;
        constexpr float kC0 = 4194304.0f + 32.0f + 256.0f * 32.0f;
        f32x4 c = f32x4{kC0, kC0, kC0, kC0};
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bq, c, 4, 4, 0, scale_a, 0, 127);
        // (elements copied out first: a bit cast of a vector element reads element 0)
        const float c0 = c[0], c1 = c[1], c2 = c[2], c3 = c[3];
        auto dots = [&](float ce, float& lo, float& hi) {
          const uint32_t bits = __builtin_bit_cast(uint32_t, ce);
          lo = 64.0f - (float)(bits & 0xffu);  // (v_cvt_f32_ubyte0)
          hi = 64.0f - (float)((bits >> 8) & 0xffu);
        };
        dots(c0, dotf[0], dotf[4]);
        dots(c1, dotf[1], dotf[5]);
        dots(c2, dotf[2], dotf[6]);
        dots(c3, dotf[3], dotf[7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        const float b = BIAS ? (b2 ? bias2d_lookup(biasw, qb2, kposs[j]) : brow[j]) : 0.0f;
        // the canonical order t = aq ak, u = t dot, v = u / sqrt(d), l = v + B (dot exact in fp32)
        float l = __fadd_rn(__fmul_rn(__fmul_rn(__fmul_rn(aqv, akk[j]), dotf[e]), a.isd), b);
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
        // (v_exp_f32 alone: the argument is a logit minus the row maximum, so a result
        // below 2^-126 that flushes to 0 is negligible beside the maximum's own 1)
        const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(lg[ks][e], log2e, -mb));
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
      const float sc = FUSED ? vsc[c] : a.vscale[(size_t)bh * D + c];
      const int cs = 128 * colsum[c];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int orow = tile * 16 + 4 * kg + r;
        if (orow < n)
          a.out[((size_t)bh * n + orow) * D + c] = div255_rn(__fmul_rn((float)(acc[nt][r] + cs), sc));
      }
    }
  }
}

template <int NK, int D, bool FUSED>
hipError_t launch_nkd(const DenseKArgs& ka, int64_t BH, hipStream_t s) {
  if constexpr (!FUSED) {
    if (ka.brow2 != nullptr) {
      const size_t lds = sizeof(float) * (bias2d_floats(ka.gh, ka.gw, ka.cls) + 32 * NK);
      hipLaunchKernelGGL((dense_q8_kernel<NK, true, D, false, true>), dim3((unsigned)BH), dim3(64 * kWaves), lds, s,
                         ka);
      return hipGetLastError();
    }
  }
  if (ka.bias != nullptr) {
    const size_t lds = sizeof(float) * (2 * ka.n - 1 + 32 * NK);
    hipLaunchKernelGGL((dense_q8_kernel<NK, true, D, FUSED>), dim3((unsigned)BH), dim3(64 * kWaves), lds, s, ka);
  } else {
    hipLaunchKernelGGL((dense_q8_kernel<NK, false, D, FUSED>), dim3((unsigned)BH), dim3(64 * kWaves), 0, s, ka);
  }
  return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_n(const DenseKArgs& ka, int d, int64_t BH, hipStream_t s) {
  const int nk = (ka.n + 31) / 32;
  auto go = [&](auto NKc) {
    constexpr int NK = decltype(NKc)::value;
    return d == 128 ? launch_nkd<NK, 128, FUSED>(ka, BH, s) : launch_nkd<NK, 64, FUSED>(ka, BH, s);
  };
  switch (nk) {
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    case 3: return go(std::integral_constant<int, 3>{});
    case 4: return go(std::integral_constant<int, 4>{});
    case 5: return go(std::integral_constant<int, 5>{});
    case 6: return go(std::integral_constant<int, 6>{});
    case 7: return go(std::integral_constant<int, 7>{});
    default: return go(std::integral_constant<int, 8>{});
  }
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
  ka.brow2 = p.brow;
  ka.bcol2 = p.bcol;
  ka.bcls2 = p.bcls;
  ka.gh = p.gh;
  ka.gw = p.gw;
  ka.cls = p.cls;
  ka.vq = static_cast<const int8_t*>(p.v);
  ka.vscale = p.vscale;
  ka.out = p.out;
  ka.H = (int)p.H;
  ka.n = (int)p.n;
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  return launch_n<false>(ka, (int)p.d, p.B * p.H, s);
}

hipError_t launch_dense_q8_fused(const DenseFusedParams& p, hipStream_t s) {
  if ((p.d != 64 && p.d != 128) || p.n > dense_q8_max_n()) return hipErrorInvalidValue;
  DenseKArgs ka{};
  ka.bias = p.bias;
  ka.out = p.out;
  ka.H = (int)p.H;
  ka.n = (int)p.n;
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  ka.xq = p.q;
  ka.xk = p.k;
  ka.xv = p.v;
  ka.qk_bf16 = p.qk_dtype == HAD_BF16;
  ka.v_bf16 = p.v_dtype == HAD_BF16;
  ka.mean = p.mode == HAD_MEAN_SIGN;
  return launch_n<true>(ka, (int)p.d, p.B * p.H, s);
}

}  // namespace had
