// Top-N binarized attention with integer logits (alpha = 1, no bias) and bf16
// V, for n <= 1024: distances and A*V on the matrix cores, exact top-N
// selection on VALU.
//
// Method (Hamming Attention Distillation, summary "main points"/"method";
// BinaryAttention sections 2.2-2.3):
//   l_ij = (d - 2 h_ij) / sqrt(d),  h_ij = popcount(q_i XOR k_j)
//   S_i  = the N largest l_ij, ties to the lower j
//   O_i  = sum_{j in S_i} softmax_S(l)_j V_j                  (fp32)
// With alpha = 1 and no bias the logit is a function of h alone, so S_i is
// { h < tau } plus the lowest-indexed keys at h = tau, where tau is the
// smallest level with #{h <= tau} >= N; and the softmax weight relative to the
// threshold is w(tau - h) = exp(2 (tau - h) / sqrt(d)), a table of 65 values.
//
// Work decomposition.  A wave owns a tile of 16 queries of one (batch, head).
// Lane l serves query row r = l % 16 and key quarter g = l / 16 (keys
// [g Q, (g+1) Q), Q = n_pad / 4): the same (row, key) split as the A operand
// of v_mfma_f32_16x16x32_bf16, so no data moves between selection and the
// matrix cores.
//   1. Hamming distances on fp4 matrix cores: the workgroup expands the head's
//      key codes once into LDS as fp4 operands (-x/2), each wave multiplies them
//      by its queries (+-1) with v_mfma_scale_f32_16x16x128_f8f6f4, two key
//      blocks per product (the second scaled by 2^8), and byte permutes pack
//      the exact distances four to a register.
//   2. Threshold: per-lane counts from sums of absolute differences (v_sad_u8,
//      four keys per instruction) summed over the query's four lanes, starting
//      from a guess, bracketing and bisecting.
//   3. Ties: each lane takes its share of the keys at tau, lowest j first
//      (exclusive prefix over the four quarters, then a running count over the
//      lane's keys in ascending order).
//   4. Weights: index byte = h - tau + 65 (plus 128 for a key at tau that is
//      not taken) into an LDS table of w split as bf16 hi + bf16 lo
//      (hi = rne(w), lo = rne(w - hi): 16 significant bits), zero for h > tau.
//   5. A*V: the masked weight row of the tile (16 queries x 32 keys per step)
//      times V (exact in bf16), hi and lo into one fp32 accumulator; a
//      constant all-ones operand accumulates the softmax normaliser Z in the
//      same layout, and O = acc / Z.  V rows reach LDS by direct-to-LDS loads
//      in their natural layout (one round of keys ahead, two buffers) and the
//      B operands come out of LDS through transposing reads.
// The selection is exact (bit-identical index sets); the weights carry a
// relative error below 2^-16, far inside the fp32 output tolerance.
#include <float.h>
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

constexpr int kD = 64;
constexpr uint32_t kC = 0x01010101u;
constexpr uint32_t kM = 0x80808080u;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct MfmaKArgs {
  const uint32_t* qbits;  // [BH, n, 2]
  const uint32_t* kbits;  // [BH, n, 2]
  const uint32_t* v;      // bf16 [BH, n, 64], read as pairs
  float* out;             // [BH, n, 64]
  int32_t* idx;           // [BH, n, keep] or null
  int n, keep;
  int tiles;  // 16-query tiles per head
  int split;  // workgroups per head (four tiles each)
  int t0;     // first threshold guess
  float exp_c;  // 2 / sqrt(d) * log2(e)
};

// Value of lane S of this lane's 16-lane row (DPP row_newbcast; folds into the
// consuming VALU instruction).
template <int S>
HAD_DEVICE uint32_t row_bcast(uint32_t x) {
  // every lane reads a valid source lane, so no "old" value is needed
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + S, 0xf, 0xf, true);
}

template <int N>
struct Seq {
  template <class F>
  HAD_DEVICE static void run(F&& f) {
    Seq<N - 1>::run(f);
    f(std::integral_constant<int, N - 1>{});
  }
};
template <>
struct Seq<0> {
  template <class F>
  HAD_DEVICE static void run(F&&) {}
};

// Sum over the four lanes of one query row (lanes r, r+16, r+32, r+48).
HAD_DEVICE int quad_rows_sum(int v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// Exclusive prefix over the key quarters g = 0..3 of one query row.
HAD_DEVICE int quad_rows_excl(int v, int g) {
  const int lane = (int)lane_id();
  int a = __shfl(v, (lane - 16) & 63, 64);
  int s = v + (g >= 1 ? a : 0);
  a = __shfl(s, (lane - 32) & 63, 64);
  s += (g >= 2 ? a : 0);
  return s - v;
}

// x (below 256) in every byte: one byte permute instead of a quarter-rate multiply
HAD_DEVICE uint32_t byte_bcast(uint32_t x) { return __builtin_amdgcn_perm(0u, x, 0u); }

// Counts of this lane's keys with h <= t, from sums of absolute differences:
// with S(x) = sum over the lane's keys of |h - x| (v_sad_u8, four byte-packed
// distances per instruction), |h - (t+1)| - |h - t| is +1 for h <= t and -1
// otherwise, so #{h <= t} = (S(t+1) - S(t) + N) / 2 for N keys.  All terms are
// exact small integers.
template <int NW>
HAD_DEVICE uint32_t lane_sad(const uint32_t (&P)[NW], uint32_t x) {
  const uint32_t xb = byte_bcast(x);
  uint32_t acc = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) acc = __builtin_amdgcn_sad_u8(P[w], xb, acc);
  return acc;
}

// x + (x << 8) + (x << 16) + (x << 24), as two shift-adds: the compiler would
// otherwise fold the sum into a quarter-rate v_mul_lo_u32.
HAD_DEVICE uint32_t byte_prefix(uint32_t x) {
  uint32_t y, z;
  asm("v_lshl_add_u32 %0, %1, 8, %1" : "=v"(y) : "v"(x));
  asm("v_lshl_add_u32 %0, %1, 16, %1" : "=v"(z) : "v"(y));
  return z;
}

// (a ^ b) + c in one instruction (the compiler would rewrite ~((a ^ b) + c) as a
// subtraction and a separate xor)
HAD_DEVICE uint32_t xor_add(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t y;
  asm("v_xad_u32 %0, %1, %2, %3" : "=v"(y) : "v"(a), "v"(b), "s"(c));
  return y;
}

HAD_DEVICE uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Work decomposition over the GPU: a workgroup of four waves (one per SIMD)
// takes four consecutive tiles of one head; several workgroups share a CU.
// V of the head passes through LDS in rounds of KR keys per quarter (4 KR
// rows of 128 bytes), double-buffered: the rows of round r + 1 are requested
// when round r starts, so a workgroup needs little LDS and the loads overlap
// the work.
constexpr int kWaves = 4;
constexpr int round_keys(int nk) { return nk >= 4 ? 32 : 8 * nk; }  // KR
constexpr int round_bytes(int nk) { return 4 * round_keys(nk) * 128; }
constexpr int v_buffers(int nk) { return 8 * nk > round_keys(nk) ? 2 : 1; }

// V rows in LDS.  Row lk = g KR + kk of a round buffer holds key g KG + rr KR
// + kk (quarter g) in 128 bytes; its 32-byte channel block b (channels 16 b ..
// 16 b + 15) sits at block position b ^ vswz(lk), vswz(lk) = (g + lk) mod 4.  A
// transposing read of the B operand (each group of 16 lanes reads rows
// g KR + 8c + e0 + 0..3 of one block) then finds its four rows in four different
// 32-byte bank windows, and the groups of two quarters in eight: no bank conflicts
// with 32 banks of 4 bytes or with 64.  The direct-to-LDS loads write whole rows in
// order.
HAD_DEVICE uint32_t vswz(uint32_t g, uint32_t lk) { return (g + lk) & 3u; }

// s_waitcnt with vmcnt(0) only (expcnt and lgkmcnt left at their maxima)
HAD_DEVICE void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// IDX: also write the kept-index list (a separate instance, so that the common
// kernel carries none of its code).
template <int NK, bool PAD, bool IDX>
__global__ __launch_bounds__(64 * kWaves) void topn_mfma_kernel(const MfmaKArgs a) {
  constexpr int KG = 8 * NK;            // keys per lane quarter
  constexpr int KR = round_keys(NK);    // keys per quarter and round
  constexpr int R = KG / KR;            // rounds
  constexpr int NKR = KR / 8;           // 32-key MFMA steps per round
  constexpr int NW = 2 * NK;            // byte-packed distance words per lane
  constexpr int RB = round_bytes(NK);   // bytes of one round buffer
  static_assert(R * KR == KG && KR % 8 == 0, "rounds must tile the quarter");
  constexpr int NP = 32 * NK;           // padded keys
  constexpr int KQB = KG * 32;          // bytes of fp4 operands per key quarter
  constexpr int VB = (RB > 2 * KQB + 256 ? RB : 2 * KQB + 256);  // bytes per LDS buffer
  // Static LDS arrays, at addresses fixed at compile time (a lookup address is
  // index * 4 plus an immediate offset): the weight table and the byte -> eight
  // fp4 nibble tables of the codes.
  __shared__ __align__(16) uint32_t tab[256];
  __shared__ __align__(16) uint32_t one_pairs[4];  // bf16 (1, 1) pairs: the all-ones B operand
  __shared__ __align__(16) uint32_t lut_k[256];  // key bits -> -x/2: bit 1 (x = -1) -> +0.5 (0x1), else -0.5 (0x9)
  __shared__ __align__(16) uint32_t lut_q[256];  // query bits -> x: bit 1 -> -1.0 (0xA), else +1.0 (0x2)
  // Two buffers: first the fp4 key operands (quarters 0, 1 in the first, 2, 3 in
  // the second), then the V rows of alternate rounds.  Separate arrays, so that the
  // compiler can tell the round being read from the round being loaded.
  __shared__ __align__(16) uint8_t vbuf0[VB];
  __shared__ __align__(16) uint8_t vbuf1[VB];
  auto vbuf = [&](int rr) { return (lds_u8*)((rr & 1) ? vbuf1 : vbuf0); };
  // Quarter q of the fp4 key operands starts at an LDS address of 16 (q & 1) + 128 (q >> 1)
  // modulo 256: the 16 lanes of a K-block then read four 16-byte slots of each quarter
  // that together cover every bank once (64 banks of 4 bytes), or twice (32 banks).
  auto kxq = [&](int quarter) {
    lds_u8* const b = (lds_u8*)(quarter >= 2 ? vbuf1 : vbuf0) + (quarter & 1) * KQB;
    const uint32_t want = 16u * (uint32_t)(quarter & 1) + 128u * (uint32_t)(quarter >> 1);
    return b + ((want - (uint32_t)(uintptr_t)b) & 255u);
  };

  __builtin_amdgcn_s_setprio(3);
  const int lane = (int)lane_id();
  const int g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = a.n, keep = a.keep;
  // logical workgroup ids are XCD-major, so the workgroups of one head share an
  // XCD's L2 (hardware workgroup w runs on XCD w % 8)
  const int wg = (int)xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.split;                 // the head
  const int t = (wg % a.split) * kWaves + wave;  // this wave's tile
  const bool have = t < a.tiles;                       // wave-uniform
  const size_t hb = (size_t)bh * n;
  const int i = t * 16 + r;  // this lane's query

  // ---- V rows into LDS.  Wave w loads the KR rows of quarter w of a round, eight
  // rows per instruction (lane l: row 8 m + l / 8, 16-byte piece l % 8, i.e. block
  // (l % 8) / 2 ^ vswz, half l % 2).  Padding keys load row n - 1: their weights are 0.
  const uint16_t* vh = reinterpret_cast<const uint16_t*>(a.v) + hb * kD;
  const uint32_t lrow = (uint32_t)lane >> 3;
  const uint32_t piece = (uint32_t)lane & 7u;
  const uint32_t vcol = 16u * (((piece >> 1) ^ vswz((uint32_t)wave, lrow))) + 8u * (piece & 1u);
  // (the row part of the address is wave-uniform: a scalar base plus this lane's
  // 32-bit offset, so the loads cost no vector address arithmetic)
  const uint32_t lane_off = lrow * 128u + vcol * 2u;
  auto issue_round = [&](int rr) {
    lds_u8* buf = vbuf(rr) + wave * KR * 128;
#pragma unroll
    for (int m = 0; m < KR / 8; ++m) {
      const int key0 = wave * KG + rr * KR + 8 * m;  // this instruction's first row
      const char* src;
      if (PAD) {
        const int key = min(key0 + (int)lrow, n - 1);
        src = reinterpret_cast<const char*>(vh) + (size_t)key * (kD * 2) + vcol * 2u;
      } else {
        src = reinterpret_cast<const char*>(vh) + (size_t)key0 * (kD * 2) + lane_off;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + m * 1024), 16, 0, 0);
    }
  };
  // ---- tables: softmax weights, and the fp4 nibbles of code bytes
  for (int e = threadIdx.x; e < 256; e += 64 * kWaves) {
    uint32_t ent = 0u;
    if (e >= 1 && e <= 65) {
      const float w = exp2f((float)(65 - e) * a.exp_c);  // w(tau - h), h = e + tau - 65
      const uint32_t hi16 = bf16_rne_bits(w);
      const float rest = w - __builtin_bit_cast(float, hi16 << 16);
      ent = hi16 | (bf16_rne_bits(rest) << 16);
    }
    tab[e] = ent;
    if (e < 4) one_pairs[e] = 0x3f803f80u;
    // bit b of e to bit 4b (three shift-or-mask steps), then to bit 3 of nibble b:
    // a set code bit turns 0x9 (-0.5) into 0x1 (+0.5) for keys, 0x2 (+1) into 0xA (-1)
    // for queries
    uint32_t sp = (uint32_t)e;
    sp = (sp | (sp << 12)) & 0x000f000fu;
    sp = (sp | (sp << 6)) & 0x03030303u;
    sp = (sp | (sp << 3)) & 0x11111111u;
    lut_k[e] = 0x99999999u ^ (sp << 3);
    lut_q[e] = 0x22222222u ^ (sp << 3);
  }
  // the codes: the query of this lane, and the keys this thread expands (loaded
  // before any direct-to-LDS load, whose presence makes every wait a full wait)
  const uint2 q = reinterpret_cast<const uint2*>(a.qbits)[hb + min(i, n - 1)];
  const uint2* kb = reinterpret_cast<const uint2*>(a.kbits) + hb;
  constexpr int KU = (NP + 64 * kWaves - 1) / (64 * kWaves);  // keys per thread
  uint2 kc[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int j = min((int)threadIdx.x + u * 64 * kWaves, NP - 1);
    kc[u] = kb[PAD ? min(j, n - 1) : j];  // padding keys: any code (their distances are overwritten)
  }
  __syncthreads();
  // ---- fp4 operands of every key of the head: key j = g' KG + k goes to quarter
  // g' at k * 32: dims 0-31 in bytes 0-15, dims 32-63 in bytes 16-31
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int j = (int)threadIdx.x + u * 64 * kWaves;
    if (NP % (64 * kWaves) == 0 || j < NP) {
      const uint2 c = kc[u];
      lds_u32x4* dst = (lds_u32x4*)(kxq(j / KG) + (j % KG) * 32);
      dst[0] = u32x4{lut_k[c.x & 0xffu], lut_k[(c.x >> 8) & 0xffu], lut_k[(c.x >> 16) & 0xffu], lut_k[c.x >> 24]};
      dst[1] = u32x4{lut_k[c.y & 0xffu], lut_k[(c.y >> 8) & 0xffu], lut_k[(c.y >> 16) & 0xffu], lut_k[c.y >> 24]};
    }
  }
  __syncthreads();

  uint32_t P[NW];
  int tau = 0, less = 0, cl_lo = 0, cl_hi = 0;
  if (have) {
    // ------------------------------------------------ 1. Hamming distances on the matrix cores
    // v_mfma_scale_f32_16x16x128_f8f6f4 on fp4 operands: column r of B is query r as
    // +-1 in all four K-blocks, and row rho of A holds two blocks of keys: K-blocks
    // 0, 1 the 64 dims of key (rho / 4) KG + 4b + rho % 4 as -x/2, K-blocks 2, 3 those
    // of the same key of block b + 1, the latter scaled by 2^8 (the per-block E8M0
    // scale of A).  From C = 2^22 + 32 + 256 * 32, the product is
    //   C = 2^22 + h(b) + 256 h(b + 1)
    // exactly: every partial sum is a multiple of 1/2 below 2^23, where fp32 steps by
    // 1/2.  The float's bits are then 0x4A800000 + 2 h(b) + 512 h(b + 1): byte 0
    // holds 2 h(b) and byte 1 holds 2 h(b + 1).  One LDS read and one product give
    // the distances of two key blocks; byte permutes gather them and a shift halves
    // them.  Lane (g, r) ends with the distances of query r to keys g KG + 4b + 0..3:
    // one byte-packed word P[b].
    const uint32_t qw = (g & 1) ? q.y : q.x;
    v8i Bq;
    Bq[0] = (int)lut_q[qw & 0xffu];
    Bq[1] = (int)lut_q[(qw >> 8) & 0xffu];
    Bq[2] = (int)lut_q[(qw >> 16) & 0xffu];
    Bq[3] = (int)lut_q[qw >> 24];
    Bq[4] = Bq[5] = Bq[6] = Bq[7] = 0;
    const int scale_a = g >= 2 ? 127 + 8 : 127;  // E8M0: 2^8 for block b + 1
    const lds_u8* ka = kxq(r >> 2) + (r & 3) * 32 + (g & 1) * 16 + (g >> 1) * 128;
    // four independent products (eight key blocks) in flight before any result is read
    constexpr int G = NW < 8 ? NW : 8;
    static_assert(NW % 2 == 0 && G % 2 == 0, "key blocks come in pairs");
    constexpr float kC0 = 4194304.0f + 32.0f + 256.0f * 32.0f;
#pragma unroll
    for (int b0 = 0; b0 < NW; b0 += G) {
      f32x4 c[G / 2];
#pragma unroll
      for (int j = 0; j < G / 2; ++j) {
        const u32x4 av = *(const lds_u32x4*)(ka + (b0 + 2 * j) * 128);
        v8i A;
        A[0] = (int)av[0]; A[1] = (int)av[1]; A[2] = (int)av[2]; A[3] = (int)av[3];
        A[4] = A[5] = A[6] = A[7] = 0;
        c[j] = f32x4{kC0, kC0, kC0, kC0};
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bq, c[j], 4, 4, 0, scale_a, 0, 127);
      }
#pragma unroll
      for (int j = 0; j < G / 2; ++j) {
        // (elements copied out first: a bit cast of a vector element reads element 0)
        const float e0 = c[j][0], e1 = c[j][1], e2 = c[j][2], e3 = c[j][3];
        const uint32_t f0 = __builtin_bit_cast(uint32_t, e0), f1 = __builtin_bit_cast(uint32_t, e1);
        const uint32_t f2 = __builtin_bit_cast(uint32_t, e2), f3 = __builtin_bit_cast(uint32_t, e3);
        const uint32_t t01 = __builtin_amdgcn_perm(f1, f0, 0x05010400u);  // 2h: b.0, b.1, b+1.0, b+1.1
        const uint32_t t23 = __builtin_amdgcn_perm(f3, f2, 0x05010400u);  // 2h: b.2, b.3, b+1.2, b+1.3
        uint32_t w2[2];
        w2[0] = __builtin_amdgcn_perm(t23, t01, 0x05040100u) >> 1;  // (every byte of 2h is even)
        w2[1] = __builtin_amdgcn_perm(t23, t01, 0x07060302u) >> 1;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int b = b0 + 2 * j + h2;
          uint32_t word = w2[h2];
          if (PAD) {
            // padding keys (j >= n) get a byte of at least 65, above every real distance:
            // h | 0x41 lies in [65, 127], which keeps all byte sums below carry
            const int real = n - (g * KG + 4 * b);  // real keys in this word
            const uint32_t pm = real >= 4 ? 0u : (real <= 0 ? 0x41414141u : (0x41414141u << (8 * real)));
            word |= pm;
          }
          P[b] = word;
        }
      }
    }
  }
  // ---- every wave is done with the key operands: the V rows of rounds 0 and 1
  // replace them, while the threshold is found
  __syncthreads();
  issue_round(0);
  if (R > 1) issue_round(1);

  if (have) {
    // ------------------------------------------------ 2. threshold
    // Invariant once bracketed: C(lo) < keep <= C(hi), C(t) = #{h <= t} over the
    // query's keys; llo / lhi are this lane's share of C(lo) / C(hi).  (Written
    // as selects: conditional stores to different variables would be merged into
    // a store through a selected address, which forces them to memory.)
    const int tq = a.t0;
    int lo, hi, clo, llo, lhi;
    // sums kept at the bracket's inner edges, sl = S(lo + 1) and sh = S(hi), so that a
    // probe next to an edge needs one new sum instead of two
    int sl, sh;
    {
      const int sm = (int)lane_sad<NW>(P, (uint32_t)tq - 1u);
      const int s0 = (int)lane_sad<NW>(P, (uint32_t)tq);
      const int sp = (int)lane_sad<NW>(P, (uint32_t)tq + 1u);
      const int cx = (s0 - sm + 4 * NW) >> 1, cy = (sp - s0 + 4 * NW) >> 1;  // C(tq - 1), C(tq)
      const int both = quad_rows_sum((cy << 16) | cx);
      const int ta = both & 0xffff, tb = both >> 16;
      const bool below = ta >= keep;         // tau <= tq - 1
      const bool at = !below && tb >= keep;  // tau == tq
      lo = below ? -1 : (at ? tq - 1 : tq);
      hi = below ? tq - 1 : (at ? tq : 65);  // C(65) = n >= keep: a placeholder bound
      clo = below ? 0 : (at ? ta : tb);
      llo = below ? 0 : (at ? cx : cy);
      lhi = below ? cx : (at ? cy : 0);
      sl = sp;  // S(lo + 1) when lo = tq
      sh = sm;  // S(hi) when hi = tq - 1
    }
    while (__builtin_amdgcn_ballot_w64(hi - lo > 1) != 0) {
      // probe next to the guess first, then bisect
      const bool open = hi - lo > 1;
      int mid = hi == 65 ? lo + 1 : (lo == -1 ? hi - 1 : (lo + hi) >> 1);
      mid = open ? mid : hi;  // settled lanes re-count harmlessly
      const bool next_lo = mid == lo + 1 && lo >= 0;  // (sl is defined once lo >= 0)
      const bool next_hi = mid == hi - 1 && hi < 65 && !next_lo;  // (sh is defined once hi < 65)
      // C(mid) = (S(mid + 1) - S(mid) + count) / 2
      const int s1 = (int)lane_sad<NW>(P, (uint32_t)(next_lo ? mid + 1 : mid));
      int smid = next_lo ? sl : s1, snext = next_lo ? s1 : sh;
      if (__builtin_amdgcn_ballot_w64(open && !next_lo && !next_hi) != 0) {
        const int s2 = (int)lane_sad<NW>(P, (uint32_t)mid + 1u);
        snext = (next_lo || next_hi) ? snext : s2;
      }
      const int cm = (snext - smid + 4 * NW) >> 1;
      const int tm = quad_rows_sum(cm);
      const bool up = open && tm >= keep;  // mid becomes the upper bound
      const bool dn = open && tm < keep;   // mid becomes the lower bound
      hi = up ? mid : hi;
      lhi = up ? cm : lhi;
      sh = up ? smid : sh;
      lo = dn ? mid : lo;
      clo = dn ? tm : clo;
      llo = dn ? cm : llo;
      sl = dn ? snext : sl;
    }
    tau = hi;
    less = clo;
    cl_lo = llo;
    cl_hi = lhi;
  }
  // ---- the rows of round 0 (and 1) are in place
  wait_vmem();  // this wave's direct-to-LDS loads
  __syncthreads();

  // ------------------------------------------------ 3. ties
  const int ceq = cl_hi - cl_lo;              // this lane's keys at tau
  const int before = quad_rows_excl(ceq, g);  // keys at tau in lower quarters
  const int take = min(max(keep - less - before, 0), ceq);
  const uint32_t kidx = byte_bcast((uint32_t)(65 - tau));
  const uint32_t ktau = byte_bcast((uint32_t)tau);
  const uint32_t kcut = 127u - (uint32_t)take;

  // ------------------------------------------------ 4-5. weights and A*V
  f32x4 acc[4], accz;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  accz = f32x4{0.f, 0.f, 0.f, 0.f};
  // (read from LDS once: a constant operand would be rematerialized at every step)
  const bf16x8 ones = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(lds_u8*)one_pairs);
  // B operand of channel tile tt by two transposing reads: in each group of 16 lanes
  // (K group g), lane s points at row g KR + s / 4 (+ 8c + e0) and channels
  // 16 tt + 4 (s % 4) .. + 3; lane s then receives channel 16 tt + s of keys e0 .. e0 + 3
  const uint32_t vrow0 = (uint32_t)(g * KR + (r >> 2));
  const uint32_t vsw = vswz((uint32_t)g, vrow0);
  uint32_t voff[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) voff[tt] = vrow0 * 128u + 32u * ((uint32_t)tt ^ vsw) + 8u * (uint32_t)(r & 3);
  int run = 0;  // keys at tau met so far in this lane (ascending j)
  // optional kept-index list: this lane's keys follow those of the lower quarters
  int32_t* idst = nullptr;
  int ipos = 0;
  if (IDX) {
    ipos = quad_rows_excl(cl_lo + take, g);
    idst = a.idx + (hb + (i < n ? i : 0)) * (size_t)keep;
  }
  // One 32-key step c over the lane's keys g KG + 8c + 0..7: prep applies the tie
  // cut and reads the weight-table entries, make_a builds the A operands from them,
  // products issues the matrix-core products.  The table and B reads of a step are
  // in flight while the products of the previous step run.
  auto prep = [&](int rr, int cl, uint32_t (&ent)[8]) {
    const int c = rr * NKR + cl;
    const uint32_t P0 = P[2 * c], P1 = P[2 * c + 1];
    // keys at tau: a byte of (P ^ tau) + 0x7f has bit 7 clear exactly where h == tau
    // (every byte of P ^ tau is below 0x80, so no carry crosses a byte)
    const uint32_t E0 = ~xor_add(P0, ktau, 0x7f7f7f7fu) & kM;
    const uint32_t E1 = ~xor_add(P1, ktau, 0x7f7f7f7fu) & kM;
    const int mid = __builtin_popcount(E0) + run;
    const int run1 = __builtin_popcount(E1) + mid;
    // keys at tau not taken: all of them once the lane's count passes take, the
    // first ones of this step kept where it passes take inside the step
    const bool over = run1 > take;
    uint32_t U0 = over ? E0 : 0u, U1 = over ? E1 : 0u;
    if (over && !(run >= take)) {
      // a key at tau with inclusive rank k in its word is cut when run + k > take
      // (mid + k for the second word): byte b of byte_prefix((E >> 7) + 127 - take + run)
      // is 127 - take + run + rank_b, in [120, 134], with bit 7 set exactly then
      U0 = E0 & byte_prefix((E0 >> 7) + kcut + (uint32_t)run);
      U1 = E1 & byte_prefix((E1 >> 7) + kcut + (uint32_t)mid);
    }
    run = run1;
    // h - tau + 65 per byte, plus 128 for a key at tau that is not taken
    const uint32_t I0 = P0 + kidx + U0, I1 = P1 + kidx + U1;
    if (IDX && i < n) {
      // kept keys have a table index in [1, 65]
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint32_t ib = ((b < 4 ? I0 : I1) >> (8 * (b & 3))) & 0xffu;
        if (ib <= 65u && ipos < keep) idst[ipos++] = g * KG + 8 * c + b;
      }
    }
    // table entries (hi | lo << 16) of the eight keys
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      ent[b] = tab[(I0 >> (8 * b)) & 0xffu];
      ent[4 + b] = tab[(I1 >> (8 * b)) & 0xffu];
    }
  };
  auto loadB = [&](int rr, int cl, bf16x8 (&Bv)[4]) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      lds_u8* const ad = vbuf(rr) + voff[tt] + 8 * cl * 128;
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ad);
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ad + 4 * 128));
      Bv[tt] = __builtin_bit_cast(bf16x8, i16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
    }
  };
  auto make_a = [&](const uint32_t (&ent)[8], bf16x8& A_hi, bf16x8& A_lo) {
    uint32_t ah[4], al[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ah[e] = __builtin_amdgcn_perm(ent[2 * e + 1], ent[2 * e], 0x05040100u);
      al[e] = __builtin_amdgcn_perm(ent[2 * e + 1], ent[2 * e], 0x07060302u);
    }
    A_hi = __builtin_bit_cast(bf16x8, make_uint4(ah[0], ah[1], ah[2], ah[3]));
    A_lo = __builtin_bit_cast(bf16x8, make_uint4(al[0], al[1], al[2], al[3]));
  };
  auto products = [&](const bf16x8& A_hi, const bf16x8& A_lo, const bf16x8 (&Bv)[4]) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, Bv[tt], acc[tt], 0, 0, 0);
    accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, ones, accz, 0, 0, 0);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, Bv[tt], acc[tt], 0, 0, 0);
    accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, ones, accz, 0, 0, 0);
  };
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (rr > 0) {
      // round rr's rows have landed, and every wave is done with buffer (rr + 1) & 1
      wait_vmem();
      __syncthreads();
      if (rr + 1 < R) issue_round(rr + 1);
    }
    // Issue priority falls as a wave advances (3 in the first quarter of the rounds,
    // 0 in the last): the workgroups sharing a CU then advance together instead of
    // oldest first, and the SIMDs keep several waves to choose from to the end.
    if (rr * 4 / R == 1) __builtin_amdgcn_s_setprio(2);
    if (rr * 4 / R == 2 && (rr - 1) * 4 / R != 2) __builtin_amdgcn_s_setprio(1);
    if (rr * 4 / R == 3 && (rr - 1) * 4 / R != 3) __builtin_amdgcn_s_setprio(0);
    if (have) {
      // step cl: A operands of cl, then the tie cut and table reads of cl + 1, the
      // products of cl, and the B reads of cl + 1
      bf16x8 Bv[2][4];
      uint32_t ent[2][8];
      loadB(rr, 0, Bv[0]);
      prep(rr, 0, ent[0]);
#pragma unroll
      for (int cl = 0; cl < NKR; ++cl) {
        bf16x8 A_hi, A_lo;
        make_a(ent[cl & 1], A_hi, A_lo);
        if (cl + 1 < NKR) prep(rr, cl + 1, ent[(cl + 1) & 1]);
        products(A_hi, A_lo, Bv[cl & 1]);
        if (cl + 1 < NKR) loadB(rr, cl + 1, Bv[(cl + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);  // (keeps the next step's operand build after these reads)
      }
    }
  }
  if (!have) return;

  // ------------------------------------------------ output: rows 4g + e, channel 16 tt + r
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = t * 16 + 4 * g + e;
    const float inv = __builtin_amdgcn_rcpf(accz[e]);  // (1 ulp; Z >= 1: the weight at tau is 1)
    if (row < n) {
      float* o = a.out + (hb + row) * kD + r;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) o[16 * tt] = acc[tt][e] * inv;
    }
  }
}

template <int NK, bool PAD, bool IDX>
hipError_t launch_nk(const MfmaKArgs& ka, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((topn_mfma_kernel<NK, PAD, IDX>), grid, block, 0, s, ka);
  return hipGetLastError();
}

template <int NK>
hipError_t launch_pad(const MfmaKArgs& ka, bool pad, dim3 grid, dim3 block, hipStream_t s) {
  if (ka.idx != nullptr)
    return pad ? launch_nk<NK, true, true>(ka, grid, block, s) : launch_nk<NK, false, true>(ka, grid, block, s);
  return pad ? launch_nk<NK, true, false>(ka, grid, block, s) : launch_nk<NK, false, false>(ka, grid, block, s);
}

// Smallest t with P(Binomial(d, 1/2) <= t) >= keep / n: the expected threshold
// for codes of independent signs, a starting guess only.
int threshold_guess(int64_t d, int64_t keep, int64_t n) {
  double c = 1.0, cdf = 0.0;
  const double total = ldexp(1.0, (int)d);
  for (int t = 0; t <= d; ++t) {
    cdf += c / total;
    if (cdf >= (double)keep / (double)n) return t;
    c = c * (double)(d - t) / (double)(t + 1);
  }
  return (int)d;
}

}  // namespace

bool topn_mfma_supported(const AttnParams& p) {
  return p.d == kD && p.v_kind == 1 && p.alpha_q == nullptr && p.alpha_k == nullptr && p.bias == nullptr &&
         p.brow == nullptr && p.n >= 1 && p.n <= 1024;
}

hipError_t launch_topn_mfma(const AttnParams& p, hipStream_t s) {
  if (!topn_mfma_supported(p)) return hipErrorInvalidValue;
  int NK = 2;  // 32-key steps per lane quarter step: n_pad = 32 NK (NK even)
  while (32 * NK < p.n) NK *= 2;
  MfmaKArgs ka{};
  ka.qbits = p.qbits;
  ka.kbits = p.kbits;
  ka.v = static_cast<const uint32_t*>(p.v);
  ka.out = p.out;
  ka.idx = p.idx;
  ka.n = (int)p.n;
  ka.keep = (int)p.keep;
  ka.tiles = (int)((p.n + 15) / 16);
  ka.t0 = std::max(1, threshold_guess(p.d, p.keep, p.n));
  ka.exp_c = (float)(2.0 / sqrt((double)p.d) * 1.4426950408889634);
  const int64_t BH = p.B * p.H;
  ka.split = (ka.tiles + kWaves - 1) / kWaves;
  if (BH * ka.split >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(BH * ka.split));
  const dim3 block((unsigned)(64 * kWaves));
  const bool pad = p.n != 32 * NK;
  switch (NK) {
    case 2: return launch_pad<2>(ka, pad, grid, block, s);
    case 4: return launch_pad<4>(ka, pad, grid, block, s);
    case 8: return launch_pad<8>(ka, pad, grid, block, s);
    case 16: return launch_pad<16>(ka, pad, grid, block, s);
    default: return launch_pad<32>(ka, pad, grid, block, s);
  }
}

}  // namespace had
