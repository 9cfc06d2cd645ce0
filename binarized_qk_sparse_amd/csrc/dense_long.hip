// BinaryAttention forward for sequences longer than one workgroup holds on chip:
// dense softmax over all keys, uint8 A times per-channel int8 V on the int8
// matrix cores, keys streamed through LDS in tiles.
//
// BinaryAttention, section 2.3 (Softmax(QK^T/sqrt(d) + B) V with QK^T from the
// binarized codes of section 2.2) and section 2.4 (mixed quantization):
//   A_q = clamp(rint(255 p), 0, 255),  O = float(sum_j A_q[j] Vq[j][c]) * scale[c] / 255.
// A_q needs p normalised over the whole row before any key's A_q is known, so
// the kernel makes two passes over the keys: the first finds each row's maximum
// logit and the sum of exp(l - max) (per lane online, the running sum rescaled
// when the maximum rises), the second recomputes the logits, quantizes A and
// contracts it with the int8 V tile.  Recomputing the logits (XOR + popcount and
// a few float ops per pair) costs less than storing them.
//
// Work split: a workgroup of four waves takes 64 queries of one (batch, head);
// wave w owns queries 16 w .. 16 w + 15.  v_mfma_i32_16x16x64_i8 layouts:
//   A (16 queries x 64 keys): lane l holds row l % 16, keys 16 (l / 16) + 0..15
//   B (64 keys x 16 channels): lane l holds channel l % 16, the same 16 keys
//   C (16 x 16 int32): lane l, element r: row 4 (l / 16) + r, channel l % 16.
// Each lane computes the logits of exactly the A elements it feeds.  The
// product only needs A and B to assign keys to lanes and bytes the same way,
// which they do.  gfx950 has no unsigned-by-signed int8 product, so A' =
// A_q - 128 is fed as int8 and 128 * sum_j Vq[j][c] is added back, exact in
// int32 (each of the two terms stays below 128 * 127 * 65536 < 2^31).
#include <float.h>

#include <type_traits>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Bit b of a code byte to bit 3 of nibble b: the key operand of the fp4 distance products
// is 0x9 (-0.5) xor this, a set bit (x = -1) giving 0x1 (-x/2 = +0.5); the query's is
// 0x2 (+1) xor this, a set bit giving 0xA (-1).
HAD_DEVICE uint32_t fp4_spread(uint32_t byte) {
  uint32_t sp = byte;
  sp = (sp | (sp << 12)) & 0x000f000fu;
  sp = (sp | (sp << 6)) & 0x03030303u;
  sp = (sp | (sp << 3)) & 0x11111111u;
  return sp << 3;
}

// Byte offset of the 16-byte half h (dims 32 h .. 32 h + 31) of key kk (0..63) of a tile
// among its fp4 operands: lane group g's sixteen keys take 512 bytes, a key's halves sit
// at slots 2 (kk % 16) + h, and group g flips slot bits 0 and 3 by g, so that the 16
// lanes of one K-block (four groups by four keys) read 16 different 16-byte slots.
HAD_DEVICE uint32_t fp4_key_offset(uint32_t kk, uint32_t h) {
  const uint32_t q = kk >> 4;
  const uint32_t slot = (2u * (kk & 15u) + h) ^ ((q & 1u) | ((q >> 1) << 3));
  return q * 512u + slot * 16u;
}

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

// Head_dim 128: byte offset of K-block b (dims 32 b .. 32 b + 31) of key kk, 64 bytes a key,
// the block index flipped by the key's lane group kk / 16 so that the 16 lanes of a K-block
// (four groups by four keys) read 16 different 16-byte slots.
HAD_DEVICE uint32_t fp4_key_offset128(uint32_t kk, uint32_t b) {
  return (kk * 4u + (b ^ ((kk >> 4) & 3u))) * 16u;
}

constexpr int kQB = 64;          // queries per workgroup (four waves of 16)
constexpr int kKT = 64;          // keys per tile
constexpr int kVRow = kKT + 16;  // bytes per channel row of the transposed int8 V tile
constexpr int kTab2d = 4096;     // floats of two-dimensional bias tables staged per workgroup

struct DenseLongArgs {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const float* aq;
  const float* ak;
  const float* bias;  // 1-D table [H, 2n - 1]
  const int8_t* vq;
  const float* vscale;
  float* out;
  int H, n, qblocks;
  float isd;
  // two-dimensional decomposable bias (BIAS == 2)
  const float* brow2;
  const float* bcol2;
  const float* bcls2;
  int gh, gw, cls;
};

// Max / sum of a row whose values live in lanes l, l^16, l^32, l^48.
HAD_DEVICE float row4_max_f(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
HAD_DEVICE float row4_sum_f(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// 2^x by v_exp_f32 alone, without the denormal-range scaling of exp2f.  Every
// argument here is a logit minus a running or final row maximum (scaled), so at
// most a rounding error above 0; a result below 2^-126 that flushes to 0 is
// negligible beside the maximum's own term, which is 1.
HAD_DEVICE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte offset of key column k (0..63) of channel row c in the transposed V tile.
// The four 16-byte chunks of a row are rotated by (c / 16) mod 4: one B-operand
// read (16 consecutive rows, one chunk each) keeps its 80-byte row stride, which
// already spreads 16 rows over all banks, and the stores of the staging pass
// (rows 16 apart land on the same banks) move to different chunks.
HAD_DEVICE int vt_off(int c, int k) { return c * kVRow + ((((k >> 4) ^ (c >> 4)) & 3) << 4) + (k & 15); }

// BIAS: 0 none, 1 the 1-D offset table, 2 the two-dimensional decomposable bias.
// ALPHA: scales present (either pointer non-null).
template <int D, bool ALPHA, int BIAS>
__global__ __launch_bounds__(256) void dense_long_kernel(const DenseLongArgs a) {
  constexpr int NT = D / 16;                  // channel tiles
  constexpr int VI = kKT * (D / 4) / 4 / 256;  // 4 x 4 byte blocks of a V tile per thread
  static_assert(VI >= 1 && VI * 256 * 16 == kKT * D, "sixteen bytes per block, every block staged");
  __shared__ __align__(16) Code<D> kc[kKT];
  // the tile's keys as fp4 operands of the distance products (32 bytes a key at head_dim 64, 64 at 128)
  __shared__ __align__(256) uint8_t kx[kKT * (D / 2)];
  __shared__ __align__(16) float akk[kKT];
  __shared__ __align__(16) float bwin[kKT + kQB];  // 1-D: bias window; 2-D: key position codes
  __shared__ __align__(16) int8_t vqt[D * kVRow];
  __shared__ int colsum[D];
  extern __shared__ float tab[];  // two-dimensional bias tables

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  // logical workgroup ids are XCD-major, so the workgroups of one head share an L2
  const int wg = (int)xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.qblocks, i0 = (wg % a.qblocks) * kQB;
  const int hh = bh % a.H, n = a.n;
  const int i = i0 + 16 * wave + r16;  // this lane's query (may be padding)
  const int iq = i < n ? i : n - 1;
  const size_t hb = (size_t)bh * n;
  const Code<D> qq = load_code<D>(a.qbits, hb + iq);
  const float aqv = (ALPHA && a.aq != nullptr) ? a.aq[hb + iq] : 1.0f;
  const int ntiles = (n + kKT - 1) / kKT;
  const float log2e = 1.4426950408889634f;

  if (tid < D) colsum[tid] = 0;
  int2 qb2 = make_int2(0, 0);
  if constexpr (BIAS == 2) {
    stage_bias2d(tab, a.brow2, a.bcol2, a.bcls2, hh, a.gh, a.gw, a.cls, tid, 256);
    qb2 = bias2d_query(iq, a.gh, a.gw, a.cls);
  }
  const float* biash = BIAS == 1 ? a.bias + (size_t)hh * (2 * n - 1) : nullptr;

  // The tile sequence is the keys twice over (t < ntiles: first pass, else
  // second).  A tile goes global -> registers -> LDS; the next tile's loads are
  // issued before the current tile is processed, so they land while it runs.
  // Threads tid < 64 carry key tid's code and scale; the 1-D bias window holds
  // the table entries of offsets j - i + n - 1 for the tile's keys and the
  // workgroup's queries (zero outside the table: padding pairs only); the int8 V
  // tile (second pass only) moves as blocks of four keys by four channels.
  Code<D> pc{};
  float pa = 1.0f, pb = 0.0f;
  uint32_t pv[VI][4];
  auto tile_j0 = [&](int t) { return (t < ntiles ? t : t - ntiles) * kKT; };
  auto fetch = [&](int t) {
    const int j0 = tile_j0(t);
    // (threads kKT.. load the same codes again and expand their other 16-byte blocks:
    // two per key at head_dim 64, four at 128)
    if (tid < (D / 32) * kKT) {
      const int j = j0 + (tid & (kKT - 1));
      const int jc = j < n ? j : n - 1;
      pc = load_code<D>(a.kbits, hb + jc);
      pa = (ALPHA && a.ak != nullptr) ? a.ak[hb + jc] : 1.0f;
    }
    if constexpr (BIAS == 1) {
      if (tid < kKT + kQB - 1) {
        const int o = j0 - (i0 + kQB - 1) + n - 1 + tid;
        pb = (o >= 0 && o <= 2 * n - 2) ? biash[o] : 0.0f;
      }
    }
    if (t >= ntiles) {
#pragma unroll
      for (int u = 0; u < VI; ++u) {
        const int e = tid + 256 * u;
        const int c4 = 4 * (e % (D / 4)), jb = 4 * (e / (D / 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + jb + r;
          pv[u][r] = j < n ? *reinterpret_cast<const uint32_t*>(a.vq + (hb + j) * D + c4) : 0u;
        }
      }
    }
  };
  int cs[VI][4];  // this thread's column sums of int8 V (second pass)
#pragma unroll
  for (int u = 0; u < VI; ++u)
#pragma unroll
    for (int c = 0; c < 4; ++c) cs[u][c] = 0;
  auto store = [&](int t) {
    const int j0 = tile_j0(t);
    if (tid < kKT) {
      kc[tid] = pc;
      akk[tid] = pa;
    }
    if (tid < (D / 32) * kKT) {
      const uint32_t h = (uint32_t)tid >> 6;  // the key's block of 32 dims
      const uint32_t w = code_word_sel<D>(pc, h);
      const uint32_t off = D == 64 ? fp4_key_offset((uint32_t)tid & 63u, h) : fp4_key_offset128((uint32_t)tid & 63u, h);
      *reinterpret_cast<uint4*>(kx + off) =
          make_uint4(0x99999999u ^ fp4_spread(w & 0xffu), 0x99999999u ^ fp4_spread((w >> 8) & 0xffu),
                     0x99999999u ^ fp4_spread((w >> 16) & 0xffu), 0x99999999u ^ fp4_spread(w >> 24));
    }
    if constexpr (BIAS == 1) {
      // + 0 turns a -0 entry into +0 (as the other kernels stage the table)
      if (tid < kKT + kQB - 1) bwin[tid] = __fadd_rn(pb, 0.0f);
    }
    if constexpr (BIAS == 2) {
      if (tid < kKT)
        reinterpret_cast<uint32_t*>(bwin)[tid] = bias2d_key(min(j0 + tid, n - 1), a.gh, a.gw, a.cls);
    }
    if (t >= ntiles) {
#pragma unroll
      for (int u = 0; u < VI; ++u) {
        const int e = tid + 256 * u;
        const int c4 = 4 * (e % (D / 4)), jb = 4 * (e / (D / 4));
        const uint32_t* w = pv[u];
        // byte transpose: word c of the result holds channel c4 + c of keys jb .. jb + 3
        const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
        const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
        const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
        const uint32_t tw[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                                __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                                __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                                __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          *reinterpret_cast<uint32_t*>(&vqt[vt_off(c4 + c, jb)]) = tw[c];
          cs[u][c] = __builtin_amdgcn_sdot4((int)tw[c], 0x01010101, cs[u][c], false);
        }
      }
    }
  };

  float m_l = -INFINITY, z_l = 0.0f;  // first pass: this lane's running max and sum
  float mb = 0.0f, q255 = 0.0f;       // second pass: max * log2(e) and 255 / Z of the row
  v4i acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = v4i{0, 0, 0, 0};
  const uint32_t* kpos = reinterpret_cast<const uint32_t*>(bwin);
  const int wbase = (kQB - 1) - 16 * wave - r16;  // 1-D window index of key column 0
  // Head_dim 64: a tile's distances from two fp4 products (the encoding of the matrix-core
  // top-N kernel): in product p, row 4 g + e of A holds key 16 g + 8 p + e in K-blocks 0, 1
  // and key 16 g + 8 p + 4 + e in K-blocks 2, 3 (scaled by 2^8), column r of B query r;
  // from C = 2^22 + 32 + 256 * 32 the result is 2^22 + h0 + 256 h1 exactly, so lane (g, r)
  // finds 2h of its sixteen keys in bytes 0 and 1 of eight results: d - 2h = 64 - byte.
  // Head_dim 128: K = 128 fills a product with one key block, so four products: in
  // product p row 4 g + e holds key 16 g + 4 p + e, K-block g' its dims 32 g' ..; from
  // C = 2^22 + 64 the result is 2^22 + h and d - 2h = 2^23 + 128 - 2C, exact in one fma.
  constexpr int NPR = D == 64 ? 2 : 4;  // products per tile
  v8i Bq{};
  int scale_a = 127;
  uint32_t koff[NPR];
  {
    const uint32_t qw = code_word_sel<D>(qq, (uint32_t)(D == 64 ? (kg & 1) : kg));
#pragma unroll
    for (int b = 0; b < 4; ++b) Bq[b] = (int)(0x22222222u ^ fp4_spread((qw >> (8 * b)) & 0xffu));
    if constexpr (D == 64) scale_a = kg >= 2 ? 127 + 8 : 127;
#pragma unroll
    for (int p = 0; p < NPR; ++p)
      koff[p] = D == 64 ? fp4_key_offset((uint32_t)(16 * (r16 >> 2) + 8 * p + (r16 & 3) + 4 * (kg >> 1)), (uint32_t)(kg & 1))
                        : fp4_key_offset128((uint32_t)(16 * (r16 >> 2) + 4 * p + (r16 & 3)), (uint32_t)kg);
  }

  fetch(0);
  for (int t = 0; t < 2 * ntiles; ++t) {
    __syncthreads();  // every wave is done with the previous tile
    store(t);
    if (t + 1 < 2 * ntiles) fetch(t + 1);
    __syncthreads();
    const bool second = t >= ntiles;
    const int j0 = tile_j0(t);
    if (t == ntiles) {
      // the row's maximum and normaliser from its four lanes
      const float M = row4_max_f(m_l);
      const float zr = row4_sum_f(z_l * fast_exp2(__builtin_fmaf(m_l, log2e, -M * log2e)));
      mb = M * log2e;
      q255 = 255.0f / zr;
    }
    // ---- logits of this lane's 16 keys (only the last tile holds padding keys)
    float l[16];
    float dotf[16];
    if constexpr (D == 128) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 av = *reinterpret_cast<const uint4*>(kx + koff[p]);
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
    }
    if constexpr (D == 64) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint4 av = *reinterpret_cast<const uint4*>(kx + koff[p]);
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
        dots(c0, dotf[8 * p + 0], dotf[8 * p + 4]);
        dots(c1, dotf[8 * p + 1], dotf[8 * p + 5]);
        dots(c2, dotf[8 * p + 2], dotf[8 * p + 6]);
        dots(c3, dotf[8 * p + 3], dotf[8 * p + 7]);
      }
    }
    auto logits = [&](auto full) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int jj = 16 * kg + e;
        const float dot = dotf[e];
        float b = 0.0f;
        if constexpr (BIAS == 1) b = bwin[jj + wbase];
        if constexpr (BIAS == 2) b = bias2d_lookup(tab, qb2, kpos[jj]);
        float lv;
        if constexpr (ALPHA) {
          // the canonical order t = aq ak, u = t dot, v = u / sqrt(d), l = v + B
          lv = __fadd_rn(__fmul_rn(__fmul_rn(__fmul_rn(aqv, akk[jj]), dot), a.isd), b);
        } else {
          // alpha = 1: the canonical product 1 * 1 * dot is dot exactly
          lv = __fadd_rn(__fmul_rn(dot, a.isd), b);
        }
        if constexpr (decltype(full)::value) {
          l[e] = lv;
        } else {
          l[e] = j0 + jj < n ? lv : -INFINITY;
        }
      }
    };
    if (j0 + kKT <= n) {
      logits(std::true_type{});
    } else {
      logits(std::false_type{});
    }
    if (!second) {
      float mx = l[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, l[e]);
      const float mn = fmaxf(m_l, mx);
      const float mnb = mn == -INFINITY ? 0.0f : mn * log2e;  // (a lane with only padding so far)
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s += fast_exp2(__builtin_fmaf(l[e], log2e, -mnb));
      z_l = __builtin_fmaf(z_l, fast_exp2(__builtin_fmaf(m_l, log2e, -mnb)), s);
      m_l = mn;
    } else {
      // v_cvt_pk_u8_f32 rounds to nearest even, clamps to [0, 255] and writes the
      // byte in place; xor 0x80 turns each A_q into A_q - 128
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e)
        w[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(fast_exp2(__builtin_fmaf(l[e], log2e, -mb)) * q255, e & 3, w[e >> 2]);
      const v4i A = v4i{(int)(w[0] ^ 0x80808080u), (int)(w[1] ^ 0x80808080u), (int)(w[2] ^ 0x80808080u),
                        (int)(w[3] ^ 0x80808080u)};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const v4i Bv = *reinterpret_cast<const v4i*>(&vqt[vt_off(nt * 16 + r16, 16 * kg)]);
        acc[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bv, acc[nt], 0, 0, 0);
      }
    }
  }

  // ---- column sums of int8 V over all keys, then dequantize and store
#pragma unroll
  for (int u = 0; u < VI; ++u) {
    const int c4 = 4 * ((tid + 256 * u) % (D / 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) atomicAdd(&colsum[c4 + c], cs[u][c]);
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = nt * 16 + r16;
    const float sc = a.vscale[(size_t)bh * D + c];
    const int cs128 = 128 * colsum[c];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int orow = i0 + 16 * wave + 4 * kg + r;
      if (orow < n) a.out[(hb + orow) * D + c] = div255_rn(__fmul_rn((float)(acc[nt][r] + cs128), sc));
    }
  }
}

template <int D, bool ALPHA, int BIAS>
hipError_t launch_dl(const DenseLongArgs& ka, int64_t BH, size_t lds, hipStream_t s) {
  const dim3 grid((unsigned)(BH * ka.qblocks));
  hipLaunchKernelGGL((dense_long_kernel<D, ALPHA, BIAS>), grid, dim3(256), lds, s, ka);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dl_d(const DenseLongArgs& ka, bool alpha, int64_t BH, hipStream_t s) {
  if (ka.brow2 != nullptr) {
    const size_t lds = sizeof(float) * (size_t)bias2d_floats(ka.gh, ka.gw, ka.cls);
    return alpha ? launch_dl<D, true, 2>(ka, BH, lds, s) : launch_dl<D, false, 2>(ka, BH, lds, s);
  }
  if (ka.bias != nullptr) return alpha ? launch_dl<D, true, 1>(ka, BH, 0, s) : launch_dl<D, false, 1>(ka, BH, 0, s);
  return alpha ? launch_dl<D, true, 0>(ka, BH, 0, s) : launch_dl<D, false, 0>(ka, BH, 0, s);
}

}  // namespace

int64_t dense_long_bias2d_max() { return kTab2d; }

hipError_t launch_dense_long(const AttnParams& p, hipStream_t s) {
  if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
  if (p.brow != nullptr && bias2d_floats(p.gh, p.gw, p.cls) > kTab2d) return hipErrorInvalidValue;
  DenseLongArgs ka{};
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
  ka.qblocks = (int)((p.n + kQB - 1) / kQB);
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  const int64_t BH = p.B * p.H;
  if (BH * ka.qblocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const bool alpha = p.alpha_q != nullptr || p.alpha_k != nullptr;
  return p.d == 128 ? launch_dl_d<128>(ka, alpha, BH, s) : launch_dl_d<64>(ka, alpha, BH, s);
}

}  // namespace had
