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
constexpr uint32_t kM = 0x80808080u;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
  // float keys: plain sign codes with a relative-position table
  const float* bias;  // [H, 2n - 1], B[i][j] = bias[h][j - i + n - 1]
  int H;
  float isd;  // float(1 / sqrt(d))
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

// The four lanes of one query row (r, r + 16, r + 32, r + 48) exchange values with
// the gfx950 permlane swaps, on the VALU: permlane16_swap of a value with itself
// gives every lane its 16-lane row pair's values (even row, odd row), and
// permlane32_swap its 32-lane half pair's (lower half, upper half).
HAD_DEVICE void row_pair(uint32_t v, uint32_t& even, uint32_t& odd) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  even = r[0];
  odd = r[1];
}
HAD_DEVICE void half_pair(uint32_t v, uint32_t& lower, uint32_t& upper) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lower = r[0];
  upper = r[1];
}

// Sum over the four lanes of one query row.
HAD_DEVICE int quad_rows_sum(int v) {
  uint32_t e, o, l, u;
  row_pair((uint32_t)v, e, o);
  half_pair(e + o, l, u);
  return (int)(l + u);
}

HAD_DEVICE float quad_rows_max(float v) {
  uint32_t e, o, l, u;
  row_pair(__builtin_bit_cast(uint32_t, v), e, o);
  const float m = fmaxf(__builtin_bit_cast(float, e), __builtin_bit_cast(float, o));
  half_pair(__builtin_bit_cast(uint32_t, m), l, u);
  return fmaxf(__builtin_bit_cast(float, l), __builtin_bit_cast(float, u));
}

// Exclusive prefix over the key quarters g = 0..3 of one query row.
HAD_DEVICE int quad_rows_excl(int v, int g) {
  uint32_t e, o, l, u;
  row_pair((uint32_t)v, e, o);
  half_pair(e + o, l, u);
  return (int)(((g & 1) ? e : 0u) + ((g & 2) ? l : 0u));
}

// The 16 largest values of two lanes' lists (each sorted in descending order), sorted
// in descending order, in both lanes: c[k] = max(A[k], B[15 - k]) holds the 16 largest
// of the union and falls then rises (a bitonic sequence), which four half-cleaner
// layers sort.  HALF: the lanes 32 apart (quarters g and g ^ 2), else 16 apart (g ^ 1).
// Equal values may come out as either of two floats that compare equal (+0 and -0),
// which leaves every count of values above or equal to a bound unchanged.
template <bool HALF>
HAD_DEVICE void pair_top16(float (&m)[16]) {
  float c[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t a0, b0, a1, b1;  // first and second lane's values at k and at 15 - k
    if constexpr (HALF) {
      half_pair(__builtin_bit_cast(uint32_t, m[k]), a0, b0);
      half_pair(__builtin_bit_cast(uint32_t, m[15 - k]), a1, b1);
    } else {
      row_pair(__builtin_bit_cast(uint32_t, m[k]), a0, b0);
      row_pair(__builtin_bit_cast(uint32_t, m[15 - k]), a1, b1);
    }
    c[k] = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, b1));
    c[15 - k] = fmaxf(__builtin_bit_cast(float, a1), __builtin_bit_cast(float, b0));
  }
#pragma unroll
  for (int j = 8; j >= 1; j >>= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & j) == 0) {
        const float hi = fmaxf(c[i], c[i + j]);
        const float lo = fminf(c[i], c[i + j]);
        c[i] = hi;
        c[i + j] = lo;
      }
#pragma unroll
  for (int k = 0; k < 16; ++k) m[k] = c[k];
}

// A sorting network on 12 inputs (39 comparators in 9 layers; every 0-1 input comes out
// sorted, which the tests check): comparator (i, j), i < j, leaves the larger value at i.
constexpr int kSort12[39][2] = {{0, 8}, {1, 7}, {2, 6}, {3, 11}, {4, 10}, {5, 9},  {0, 1}, {2, 5}, {3, 4}, {6, 9},
                                {7, 8}, {10, 11}, {0, 2}, {1, 6}, {5, 10}, {9, 11}, {0, 3}, {1, 2}, {4, 6}, {5, 7},
                                {8, 11}, {9, 10}, {1, 4}, {3, 5}, {6, 8}, {7, 10}, {1, 3}, {2, 5}, {6, 9}, {8, 10},
                                {2, 3}, {4, 5}, {6, 7}, {8, 9}, {4, 6}, {5, 7}, {3, 4}, {5, 6}, {7, 8}};

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

// Byte k of the result is 0x80 where bit k of x (x < 16) is set.
HAD_DEVICE uint32_t spread_nibble(uint32_t x) { return (((x & 0xfu) * 0x204081u) & 0x01010101u) << 7; }

// IDX: also write the kept-index list (a separate instance, so that the common
// kernel carries none of its code).
// FK (float keys): plain sign codes with a relative-position table B.  The logit
// l = fl(v(h) + T[o]) with v(h) = (d - 2h) / sqrt(d) is no longer a function of h
// alone, but when the head's table spans less than one logit step (2 / sqrt(d),
// with a margin for the rounding of the sum) every key at a level h < h' outranks
// every key at h'.  The level threshold tau is then found exactly as for integer
// logits, every key below tau is kept, and only the keys at tau need a float
// selection: the rr = N - #{h < tau} best by (l desc, j asc).  The weights are
// exp(l - v(tau) - max T) = w(tau - h) exp(T[o] - max T), a level table times a
// per-offset table, each product split into bf16 high and low parts.  Heads whose
// table spans a step or more take every key of a row as a candidate of the float
// selection and weigh each kept key by its own exp(l - max l).
template <int NK, bool PAD, bool IDX, bool FK>
__global__ __launch_bounds__(64 * kWaves) void topn_mfma_kernel(const MfmaKArgs a) {
  static_assert(!FK || NK <= 8, "float keys: up to 256 keys (a lane's keys at one level fit 64 bits)");
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
  // float keys: the head's table T[o] (o = j - i + n - 1), exp(T[o] - max T) (zero past
  // the table), the level weights w(65 - e) as floats, and the table test's partials
  __shared__ __align__(16) float ttab[FK ? 2 * NP : 1];
  __shared__ __align__(16) float wtab[FK ? 2 * NP : 1];
  __shared__ __align__(16) float ftab[FK ? 256 : 1];
  __shared__ float hred[FK ? 3 * kWaves : 1];
  // Two buffers: first the fp4 key operands (quarters 0, 1 in the first, 2, 3 in
  // the second), then the V rows of alternate rounds.  Separate arrays, so that the
  // compiler can tell the round being read from the round being loaded.
  // (256-byte aligned, so that the bank offsets of the key quarters below are
  // compile-time constants and never depend on where the compiler places them)
  __shared__ __align__(256) uint8_t vbuf0[VB];
  __shared__ __align__(256) uint8_t vbuf1[VB];
  auto vbuf = [&](int rr) { return (lds_u8*)((rr & 1) ? vbuf1 : vbuf0); };
  // Quarter q of the fp4 key operands starts at an LDS address of 16 (q & 1) + 128 (q >> 1)
  // modulo 256: the 16 lanes of a K-block then read four 16-byte slots of each quarter
  // that together cover every bank once (64 banks of 4 bytes), or twice (32 banks).
  // Both quarters of a buffer fit: quarter 0 at offset 0 or 128, quarter 1 at KQB
  // rounded up by 16 or 144 (KQB is a multiple of 256), within VB >= 2 KQB + 256.
  static_assert(KQB % 256 == 0 && VB >= 2 * KQB + 256, "fp4 key quarters and their bank offsets fit a buffer");
  auto kxq = [&](int quarter) {
    const uint32_t want = 16u * (uint32_t)(quarter & 1) + 128u * (uint32_t)(quarter >> 1);
    return (lds_u8*)(quarter >= 2 ? vbuf1 : vbuf0) + (quarter & 1) * KQB + want;
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
  // float keys: this thread's entries of the head's table, loaded with the codes
  constexpr int TPT = FK ? (2 * NP + 64 * kWaves - 1) / (64 * kWaves) : 1;  // entries per thread
  float tl[TPT];
  if constexpr (FK) {
    const float* th = a.bias + (size_t)(bh % a.H) * (2 * n - 1);
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int o = (int)threadIdx.x + u * 64 * kWaves;
      tl[u] = o < 2 * n - 1 ? th[o] : 0.0f;
    }
  }

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
    if constexpr (FK) ftab[e] = (e >= 1 && e <= 65) ? exp2f((float)(65 - e) * a.exp_c) : 0.0f;
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
  if constexpr (FK) {
    float tmin = INFINITY, tmax = -INFINITY, tnan = 0.0f;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int o = (int)threadIdx.x + u * 64 * kWaves;
      if (o < 2 * NP) ttab[o] = __fadd_rn(tl[u], 0.0f);  // (no -0 entry)
      if (o < 2 * n - 1) {
        tmin = fminf(tmin, tl[u]);
        tmax = fmaxf(tmax, tl[u]);
        tnan = tl[u] == tl[u] ? tnan : 1.0f;
      }
    }
    tmin = -wave_max_f32(-tmin);
    tmax = wave_max_f32(tmax);
    tnan = wave_max_f32(tnan);
    if (lane == 0) {
      hred[wave] = tmin;
      hred[kWaves + wave] = tmax;
      hred[2 * kWaves + wave] = tnan;
    }
  }
  __syncthreads();
  bool slow = false;  // float keys: the head's table spans a logit step or more
  if constexpr (FK) {
    float tmin = hred[0], tmax = hred[kWaves], tnan = hred[2 * kWaves];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      tmin = fminf(tmin, hred[w]);
      tmax = fmaxf(tmax, hred[kWaves + w]);
      tnan = fmaxf(tnan, hred[2 * kWaves + w]);
    }
    slow = !bias_levels_separate(tmin, tmax, tnan != 0.0f);  // uniform over the workgroup
    // exp(T - max T) for the weights of the level-ordered heads (entries past the table: 0)
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int o = (int)threadIdx.x + u * 64 * kWaves;
      if (o < 2 * NP) wtab[o] = o < 2 * n - 1 ? __expf(ttab[o] - tmax) : 0.0f;
    }
  }
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
  // ---- float keys: the exact selection (while the rows of rounds 0 and 1 land).
  // Level-ordered heads: every key below tau is kept and the row keeps the
  // rr = N - #{h < tau} best of its keys at tau by (l desc, j asc), l = fl(v(tau) +
  // T[o]); a lane caches the logits of its first twelve keys at tau and reads the
  // rest from the table on every pass.  Other heads: every real key is a candidate
  // (rr = N), its logit fl(v(h) + T[o]) formed from its distance byte.  The search
  // walks the row's distinct candidate values from the end nearer the rank (the
  // values negated when that is the low end): each round counts the values at or
  // above the current one and finds the next one below, in one pass and one pair
  // of reductions, and stops at the first value with at least rs at or above it.
  uint64_t nkb = 0;    // level-ordered heads: this lane's keys at tau that are not kept (bit p: key g KG + p)
  uint64_t keepm = 0;  // other heads: this lane's kept keys
  int kt_lane = 0;     // this lane's kept candidates
  int obase = 0;       // offset o of this lane's key g KG + p is obase + p
  float lmax = 0.0f;   // other heads: the row's largest logit
  if constexpr (FK) {
    const int iq = i < n ? i : n - 1;
    obase = g * KG - iq + n - 1;
    if (have) {
      const float vtau = __fmul_rn((float)(kD - 2 * tau), a.isd);
      const int nreal = PAD ? min(max(n - g * KG, 0), KG) : KG;  // this lane's real keys
      uint64_t cm;  // candidate bits
      if (!slow) {
        const uint32_t kt = byte_bcast((uint32_t)tau);
        cm = 0;
#pragma unroll
        for (int b = 0; b < NW; ++b) {
          const uint32_t E = ~xor_add(P[b], kt, 0x7f7f7f7fu) & kM;
          const uint32_t nib = ((E >> 7) & 1u) | ((E >> 14) & 2u) | ((E >> 21) & 4u) | (E >> 28);
          cm |= (uint64_t)nib << (4 * b);
        }
      } else {
        cm = nreal >= 64 ? ~0ull : ((1ull << nreal) - 1ull);
      }
      const int M = quad_rows_sum(__builtin_popcountll(cm));  // the row's candidates
      const int rr = slow ? keep : keep - less;               // 1 <= rr <= M
      const bool low = 2 * rr > M + 1;                        // the rank is nearer the low end
      const int rs = low ? M - rr + 1 : rr;                   // rank from the searched end
      // logit of key p of this lane's quarter (level-ordered heads: a key at tau)
      auto logit_tau = [&](int p) { return __fadd_rn(vtau, ttab[obase + p]); };
      auto logit_of = [&](uint32_t h, int p) {
        return __fadd_rn(__fmul_rn((float)(kD - 2 * (int)h), a.isd), ttab[obase + p]);
      };
      constexpr int kCache = 12;
      float bl[kCache];  // searched values of the first candidates (-inf: none)
      int bp[kCache];    // their positions p
      bool over = false;
      uint64_t rest = 0;  // candidates past the cached ones
      if (!slow) {
        rest = cm;
#pragma unroll
        for (int k = 0; k < kCache; ++k) {
          const bool has = rest != 0;
          const int p = has ? (int)__builtin_ctzll(rest) : 0;
          const float x = logit_tau(p);  // (position 0 is a valid key when there is none)
          bl[k] = has ? (low ? -x : x) : -INFINITY;
          bp[k] = p;
          rest &= rest - 1;
        }
        over = rest != 0;
      }
      // one pass over this lane's candidates y (searched domain): count(y >= t) and
      // max{y < t}
      auto scan = [&](float t, int& ge, float& below) {
        ge = 0;
        below = -INFINITY;
        auto take = [&](float y) {
          ge += y >= t ? 1 : 0;
          below = y < t ? fmaxf(below, y) : below;
        };
        if (slow) {
#pragma unroll 1
          for (int b = 0; b < NW; ++b) {
            // (a loop, recomputed on every pass: unrolled, or kept across the passes, the
            // row's logits would take a register per key, and this rarely taken path for
            // wide tables would set the register budget of every head)
            uint32_t pw = P[b];
            asm volatile("" : "+v"(pw));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int p = 4 * b + k;
              if (p < nreal) {
                const float x = logit_of((pw >> (8 * k)) & 0xffu, p);
                take(low ? -x : x);
              }
            }
          }
        } else if (!over) {
#pragma unroll
          for (int k = 0; k < kCache; ++k) take(bl[k]);  // (-inf fillers count nowhere)
        } else {
          for (uint64_t q = cm; q != 0; q &= q - 1) {
            const float x = logit_tau(__builtin_ctzll(q));
            take(low ? -x : x);
          }
        }
      };
      int ge;
      float L;
      int above = 0;  // searched values strictly above L
      bool done = false;
      bool queued = false;  // the walk below found L
      if (!slow) {
        // Walk sorted queues: each lane's twelve largest candidates in descending order.
        // Each round pops the values at or above L from the queues' heads (a few selects
        // each, instead of a pass over all cached values), counts them over the row, and
        // takes the largest remaining head as the next L.  A lane with more candidates
        // than the queue holds, whose queue runs empty before the row is done, makes
        // the wave walk again with passes over every candidate (below).
        float sq[kCache];
#pragma unroll
        for (int k = 0; k < kCache; ++k) sq[k] = bl[k];
#pragma unroll
        for (int c = 0; c < 39; ++c) {
          const float hi = fmaxf(sq[kSort12[c][0]], sq[kSort12[c][1]]);
          const float lo = fminf(sq[kSort12[c][0]], sq[kSort12[c][1]]);
          sq[kSort12[c][0]] = hi;
          sq[kSort12[c][1]] = lo;
        }
        if (over) {
          // the rest of this lane's candidates, each inserted where it belongs (the
          // smallest falls off the end)
          for (uint64_t q = rest; q != 0; q &= q - 1) {
            const float x = logit_tau(__builtin_ctzll(q));
            const float y = low ? -x : x;
#pragma unroll
            for (int k = kCache - 1; k >= 1; --k) sq[k] = fmaxf(sq[k], fminf(sq[k - 1], y));
            sq[0] = fmaxf(sq[0], y);
          }
        }
        if (__builtin_amdgcn_ballot_w64(rs > kCache) == 0) {
          // Every row's rank lies within its lanes' twelve largest values (a lane's
          // queue holds its twelve largest, and at most rs - 1 values rank above the
          // rs-th): the row's sixteen largest come from merging the four queues in two
          // pair steps, L is the one at rank rs and `above` counts those strictly above.
          float mq[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) mq[k] = k < kCache ? sq[k] : -INFINITY;
          pair_top16<false>(mq);
          pair_top16<true>(mq);
          L = mq[0];
#pragma unroll
          for (int k = 1; k < 16; ++k) L = k == rs - 1 ? mq[k] : L;
#pragma unroll
          for (int k = 0; k < 16; ++k) above += mq[k] > L ? 1 : 0;
          queued = true;
        } else {
          int popped = 0;  // this lane's values at or above L
          bool short_queue = false;  // this lane's queue ran out before its candidates did
          const int ncand = __builtin_popcountll(cm);
          L = quad_rows_max(sq[0]);  // the top value
          for (int it = 0; it <= 4 * KG && __builtin_amdgcn_ballot_w64(!done) != 0; ++it) {
            // (-inf fillers are below every L; ties pop together, one per pass.  The shift
            // is a bitwise select under an opaque mask: as a select between neighbouring
            // elements it is turned into a dynamically indexed read of the queue, a chain
            // of compares per element)
            while (__builtin_amdgcn_ballot_w64(sq[0] >= L) != 0) {
              const bool pop = sq[0] >= L;
              uint32_t m = pop ? 0xffffffffu : 0u;
              asm volatile("" : "+v"(m));
#pragma unroll
              for (int k = 0; k + 1 < kCache; ++k)
                sq[k] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, sq[k]) & ~m) |
                                                      (__builtin_bit_cast(uint32_t, sq[k + 1]) & m));
              sq[kCache - 1] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, sq[kCache - 1]) & ~m) |
                                                             (0xff800000u & m));
              popped += pop ? 1 : 0;
            }
            const int c = quad_rows_sum(popped);
            const float nb = quad_rows_max(sq[0]);  // every head is below L now
            short_queue = short_queue || (!done && popped >= kCache && ncand > kCache);
            if (!done) {
              if (c >= rs) {
                done = true;
              } else {
                above = c;
                L = nb;
              }
            }
          }
          queued = __builtin_amdgcn_ballot_w64(short_queue) == 0;
        }
      }
      if (!queued) {
        above = 0;
        done = false;
        scan(INFINITY, ge, L);
        L = quad_rows_max(L);  // the top value
        // every round moves an unfinished row one distinct value down (at most M of
        // them); the bound only guards against values the table test let through
        for (int it = 0; it <= 4 * KG && __builtin_amdgcn_ballot_w64(!done) != 0; ++it) {
          float nb;
          scan(L, ge, nb);
          const int c = quad_rows_sum(ge);
          nb = quad_rows_max(nb);
          if (!done) {
            if (c >= rs) {
              done = true;
            } else {
              above = c;
              L = nb;
            }
          }
        }
      }
      // L is the rs-th largest searched value.  In logits the threshold is L (or -L),
      // with `above` (or M - #{searched >= L}) of the row's candidates strictly above it.
      int cge, eq = 0;
      float unused;
      scan(L, cge, unused);
      const int cnt_ge = quad_rows_sum(cge);
      const int gt = low ? M - cnt_ge : above;
      const int takeq = rr - gt;  // candidates equal to the threshold that are kept, lowest j first
      // this lane's candidates equal to the threshold (per-lane branches; the prefix over
      // the row's lanes runs where every lane takes part)
      float mx = -INFINITY;
      if (slow) {
#pragma unroll 1
        for (int b = 0; b < NW; ++b)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int p = 4 * b + k;
            if (p < nreal) {
              const float x = logit_of((P[b] >> (8 * k)) & 0xffu, p);
              mx = fmaxf(mx, x);
              eq += (low ? -x : x) == L ? 1 : 0;
            }
          }
      } else if (!over) {
#pragma unroll
        for (int k = 0; k < kCache; ++k) eq += bl[k] == L ? 1 : 0;
      } else {
        for (uint64_t q = cm; q != 0; q &= q - 1) {
          const float x = logit_tau(__builtin_ctzll(q));
          eq += (low ? -x : x) == L ? 1 : 0;
        }
      }
      lmax = quad_rows_max(mx);
      int seen = quad_rows_excl(eq, g);
      // kept: above the threshold, or equal to it and among the first takeq in key order
      auto decide = [&](float y) {
        bool kept = low ? y < L : y > L;
        if (y == L) {
          kept = seen < takeq;
          ++seen;
        }
        return kept;
      };
      if (slow) {
#pragma unroll 1
        for (int b = 0; b < NW; ++b)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int p = 4 * b + k;
            if (p < nreal) {
              const float x = logit_of((P[b] >> (8 * k)) & 0xffu, p);
              if (decide(low ? -x : x)) {
                keepm |= 1ull << p;
                ++kt_lane;
              }
            }
          }
      } else if (!over) {
#pragma unroll
        for (int k = 0; k < kCache; ++k) {
          const float y = bl[k];
          if (y != -INFINITY) {
            const bool kept = decide(y);
            kt_lane += kept ? 1 : 0;
            nkb |= kept ? 0ull : (1ull << bp[k]);
          }
        }
      } else {
        for (uint64_t q = cm; q != 0; q &= q - 1) {
          const int p = __builtin_ctzll(q);
          const float x = logit_tau(p);
          if (decide(low ? -x : x)) {
            ++kt_lane;
          } else {
            nkb |= 1ull << p;
          }
        }
      }
      if (!slow) kt_lane += cl_lo;  // every key below tau
    }
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
    ipos = quad_rows_excl(FK ? kt_lane : cl_lo + take, g);
    idst = a.idx + (hb + (i < n ? i : 0)) * (size_t)keep;
  }
  // One 32-key step c over the lane's keys g KG + 8c + 0..7: prep applies the tie
  // cut and reads the weight-table entries, make_a builds the A operands from them,
  // products issues the matrix-core products.  The table and B reads of a step are
  // in flight while the products of the previous step run.
  auto prep = [&](int rr, int cl, uint32_t (&ent)[8]) {
    const int c = rr * NKR + cl;
    const uint32_t P0 = P[2 * c], P1 = P[2 * c + 1];
    if constexpr (FK) {
      if (slow) {
        // every key's own weight exp(l - max l), zero where not kept (float bits in ent)
        const uint32_t km = (uint32_t)(keepm >> (8 * c)) & 0xffu;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint32_t h = ((b < 4 ? P0 : P1) >> (8 * (b & 3))) & 0xffu;
          const float l = __fadd_rn(__fmul_rn((float)(kD - 2 * (int)h), a.isd), ttab[obase + 8 * c + b]);
          const bool kept = (km >> b) & 1u;
          ent[b] = __builtin_bit_cast(uint32_t, kept ? __expf(l - lmax) : 0.0f);
          if (IDX && kept && i < n && ipos < keep) idst[ipos++] = g * KG + 8 * c + b;
        }
        return;
      }
      // keys at tau that are not kept get + 128; the weight is the level weight times
      // exp(T[o] - max T) (float bits in ent)
      const uint32_t I0 = P0 + kidx + spread_nibble((uint32_t)(nkb >> (8 * c)) & 0xfu);
      const uint32_t I1 = P1 + kidx + spread_nibble((uint32_t)(nkb >> (8 * c + 4)) & 0xfu);
      if (IDX && i < n) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint32_t ib = ((b < 4 ? I0 : I1) >> (8 * (b & 3))) & 0xffu;
          if (ib <= 65u && ipos < keep) idst[ipos++] = g * KG + 8 * c + b;
        }
      }
      const float* wb = wtab + obase + 8 * c;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        ent[b] = __builtin_bit_cast(uint32_t, ftab[(I0 >> (8 * b)) & 0xffu] * wb[b]);
        ent[4 + b] = __builtin_bit_cast(uint32_t, ftab[(I1 >> (8 * b)) & 0xffu] * wb[4 + b]);
      }
      return;
    }
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
    if constexpr (FK) {
      // w = hi + lo: hi = bf16(w) and lo = bf16(w - hi), both rounded to nearest even
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w0 = __builtin_bit_cast(float, ent[2 * e]), w1 = __builtin_bit_cast(float, ent[2 * e + 1]);
        const bf16x2 h = {(__bf16)w0, (__bf16)w1};
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const bf16x2 lo = {(__bf16)(w0 - __builtin_bit_cast(float, hb << 16)),
                           (__bf16)(w1 - __builtin_bit_cast(float, hb & 0xffff0000u))};
        ah[e] = hb;
        al[e] = __builtin_bit_cast(uint32_t, lo);
      }
      A_hi = __builtin_bit_cast(bf16x8, make_uint4(ah[0], ah[1], ah[2], ah[3]));
      A_lo = __builtin_bit_cast(bf16x8, make_uint4(al[0], al[1], al[2], al[3]));
      return;
    }
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

// ------------------------------------------------------------------ head_dim 128
// The same decomposition at d = 128 (integer logits, bf16 V).  What changes:
//  * K = 128 fills a distance product with one key block: from C = 2^22 + 64 the
//    product of the keys (-x/2) and the queries (+-1) is C = 2^22 + h, float bits
//    0x4A800000 + 2h (partial sums are multiples of 1/2 below 2^23, so exact).  The
//    low half-words of four results are clamped to 254, gathered into bytes and
//    halved: one word of four distance bytes, levels capped at 127;
//  * the key operands (64 bytes a key) are staged in parts that fit the two buffers;
//  * with every byte below 0x80 the threshold search, the tie cut and the weight index
//    (h - tau + 127 into a table of 127 levels) work as at d = 64 whenever tau <= 126,
//    where every key at a capped level lies above tau.  A wave with a row whose
//    threshold reaches 127 recomputes its distances exactly on the VALU, finds the
//    threshold again over levels 0..128, and weighs each key on its own;
//  * A*V runs in two passes of 64 channels over the same LDS rounds (V rows staged
//    half a row at a time), the normaliser in the first.
constexpr int kD2 = 128;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int NK, bool PAD, bool IDX>
__global__ __launch_bounds__(64 * kWaves, 3) void topn_mfma_d128_kernel(const MfmaKArgs a) {
  constexpr int KG = 8 * NK;            // keys per lane quarter
  constexpr int KR = round_keys(NK);    // keys per quarter and round
  constexpr int R = KG / KR;            // rounds per channel pass
  constexpr int NKR = KR / 8;           // 32-key steps per round
  constexpr int NW = 2 * NK;            // distance words per lane
  constexpr int RB = round_bytes(NK);
  constexpr int KQB = KG * 64;                    // fp4 operand bytes per key quarter
  constexpr int NPART = 4 * KQB > 32768 ? 2 : 1;  // staging parts
  constexpr int KGP = KG / NPART;                 // keys per quarter and part
  constexpr int KQP = KQB / NPART;
  constexpr int NWP = NW / NPART;
  constexpr int VB = (RB > 2 * KQP + 64 ? RB : 2 * KQP + 64);
  static_assert(R * KR == KG && KQP % 256 == 0 && NWP % 2 == 0, "parts and rounds tile the quarter");
  __shared__ __align__(16) uint32_t tab[256];   // w(127 - e) for e in [1, 127], hi | lo << 16
  __shared__ __align__(16) uint32_t tabg[132];  // exact path: w(k) for k in [0, 128]
  __shared__ __align__(16) uint32_t one_pairs[4];
  __shared__ __align__(16) uint32_t lut_k[256];
  __shared__ __align__(16) uint32_t lut_q[256];
  __shared__ __align__(256) uint8_t vbuf0[VB];
  __shared__ __align__(256) uint8_t vbuf1[VB];
  auto vbuf = [&](int rr) { return (lds_u8*)((rr & 1) ? vbuf1 : vbuf0); };
  // quarter q of a part at 16 q bytes past a 256-byte boundary: the 16 lanes of a
  // K-block (four quarters by four keys 64 bytes apart) read 16 distinct 16-byte slots
  auto kxq = [&](int quarter) {
    return (lds_u8*)(quarter >= 2 ? vbuf1 : vbuf0) + (quarter & 1) * KQP + 16 * quarter;
  };

  __builtin_amdgcn_s_setprio(3);
  const int lane = (int)lane_id();
  const int g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = a.n, keep = a.keep;
  const int wg = (int)xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.split;
  const int t = (wg % a.split) * kWaves + wave;
  const bool have = t < a.tiles;
  const size_t hb = (size_t)bh * n;
  const int i = t * 16 + r;

  // ---- V half-rows into LDS: round rg of the two passes (channels 64 (rg / R) ..)
  const uint16_t* vh = reinterpret_cast<const uint16_t*>(a.v) + hb * kD2;
  const uint32_t lrow = (uint32_t)lane >> 3;
  const uint32_t piece = (uint32_t)lane & 7u;
  const uint32_t vcol = 16u * (((piece >> 1) ^ vswz((uint32_t)wave, lrow))) + 8u * (piece & 1u);
  const uint32_t lane_off = lrow * 256u + vcol * 2u;
  // (a wave-uniform base, made explicit, plus a 32-bit lane offset: the loads take the
  // scalar-base form and no 64-bit address per load is kept in registers)
  auto issue_round = [&](int rg) {
    const int pass = rg >= R ? 1 : 0;
    const int rr = rg - pass * R;
    lds_u8* buf = vbuf(rg) + wave * KR * 128;
#pragma unroll
    for (int m = 0; m < KR / 8; ++m) {
      const int key0 = wave * KG + rr * KR + 8 * m;
      const char* src;
      if (PAD) {
        // (the clamped offsets recomputed at every round rather than kept for all)
        uint32_t lr = lrow;
        asm volatile("" : "+v"(lr));
        const char* sb = reinterpret_cast<const char*>(vh) + __builtin_amdgcn_readfirstlane(pass * 128);
        src = sb + ((uint32_t)min(key0 + (int)lr, n - 1) * (kD2 * 2) + vcol * 2u);
      } else {
        const char* sb = reinterpret_cast<const char*>(vh) + __builtin_amdgcn_readfirstlane(key0 * (kD2 * 2) + pass * 128);
        src = sb + lane_off;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + m * 1024), 16, 0, 0);
    }
  };
  // ---- the codes: this lane's query and the keys this thread expands, every part
  const uint4 q = reinterpret_cast<const uint4*>(a.qbits)[hb + min(i, n - 1)];
  const uint4* kb = reinterpret_cast<const uint4*>(a.kbits) + hb;
  constexpr int KUP = (4 * KGP + 64 * kWaves - 1) / (64 * kWaves);  // keys per thread and part
  uint4 kc[NPART * KUP];
#pragma unroll
  for (int pt = 0; pt < NPART; ++pt)
#pragma unroll
    for (int u = 0; u < KUP; ++u) {
      const int x = min((int)threadIdx.x + u * 64 * kWaves, 4 * KGP - 1);
      const int j = (x / KGP) * KG + pt * KGP + x % KGP;
      kc[pt * KUP + u] = kb[min(j, n - 1)];  // padding keys: any code (their bytes are overwritten)
    }
  // ---- tables
  for (int e = threadIdx.x; e < 256; e += 64 * kWaves) {
    auto split = [](float w) {
      const uint32_t hi16 = bf16_rne_bits(w);
      return hi16 | (bf16_rne_bits(w - __builtin_bit_cast(float, hi16 << 16)) << 16);
    };
    tab[e] = (e >= 1 && e <= 127) ? split(exp2f((float)(127 - e) * a.exp_c)) : 0u;
    if (e <= 128) tabg[e] = split(exp2f((float)e * a.exp_c));
    if (e < 4) one_pairs[e] = 0x3f803f80u;
    uint32_t sp = (uint32_t)e;
    sp = (sp | (sp << 12)) & 0x000f000fu;
    sp = (sp | (sp << 6)) & 0x03030303u;
    sp = (sp | (sp << 3)) & 0x11111111u;
    lut_k[e] = 0x99999999u ^ (sp << 3);
    lut_q[e] = 0x22222222u ^ (sp << 3);
  }

  // ---- 1. distances, part by part
  uint32_t P[NW];
  const uint32_t qw = g == 0 ? q.x : (g == 1 ? q.y : (g == 2 ? q.z : q.w));  // dims 32 g .. 32 g + 31
  v8i Bq;
  constexpr float kC0 = 4194304.0f + 64.0f;
#pragma unroll
  for (int pt = 0; pt < NPART; ++pt) {
    __syncthreads();  // tables written (part 0); the previous part's operands read (part 1)
#pragma unroll
    for (int u = 0; u < KUP; ++u) {
      const int x = (int)threadIdx.x + u * 64 * kWaves;
      if ((4 * KGP) % (64 * kWaves) == 0 || x < 4 * KGP) {
        const uint4 c = kc[pt * KUP + u];
        lds_u32x4* dst = (lds_u32x4*)(kxq(x / KGP) + (x % KGP) * 64);
        dst[0] = u32x4{lut_k[c.x & 0xffu], lut_k[(c.x >> 8) & 0xffu], lut_k[(c.x >> 16) & 0xffu], lut_k[c.x >> 24]};
        dst[1] = u32x4{lut_k[c.y & 0xffu], lut_k[(c.y >> 8) & 0xffu], lut_k[(c.y >> 16) & 0xffu], lut_k[c.y >> 24]};
        dst[2] = u32x4{lut_k[c.z & 0xffu], lut_k[(c.z >> 8) & 0xffu], lut_k[(c.z >> 16) & 0xffu], lut_k[c.z >> 24]};
        dst[3] = u32x4{lut_k[c.w & 0xffu], lut_k[(c.w >> 8) & 0xffu], lut_k[(c.w >> 16) & 0xffu], lut_k[c.w >> 24]};
      }
    }
    if (pt == 0) {
      Bq[0] = (int)lut_q[qw & 0xffu];
      Bq[1] = (int)lut_q[(qw >> 8) & 0xffu];
      Bq[2] = (int)lut_q[(qw >> 16) & 0xffu];
      Bq[3] = (int)lut_q[qw >> 24];
      Bq[4] = Bq[5] = Bq[6] = Bq[7] = 0;
    }
    __syncthreads();
    if (have) {
      // row rho of A: key (rho / 4) KG + pt KGP + 4 b + rho % 4, K-block g of its dims
      const lds_u8* ka = kxq(r >> 2) + (r & 3) * 64 + g * 16;
      constexpr int G = NWP < 8 ? NWP : 8;
#pragma unroll
      for (int b0 = 0; b0 < NWP; b0 += G) {
        f32x4 c[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const u32x4 av = *(const lds_u32x4*)(ka + (b0 + j) * 256);
          v8i A;
          A[0] = (int)av[0]; A[1] = (int)av[1]; A[2] = (int)av[2]; A[3] = (int)av[3];
          A[4] = A[5] = A[6] = A[7] = 0;
          c[j] = f32x4{kC0, kC0, kC0, kC0};
          c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bq, c[j], 4, 4, 0, 127, 0, 127);
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float e0 = c[j][0], e1 = c[j][1], e2 = c[j][2], e3 = c[j][3];
          const uint32_t f0 = __builtin_bit_cast(uint32_t, e0), f1 = __builtin_bit_cast(uint32_t, e1);
          const uint32_t f2 = __builtin_bit_cast(uint32_t, e2), f3 = __builtin_bit_cast(uint32_t, e3);
          // low half-words (2h) of keys 0, 1 and 2, 3, clamped to 254 (level 127)
          const u16x2 cap = {254, 254};
          const u16x2 m01 = __builtin_elementwise_min(__builtin_bit_cast(u16x2, __builtin_amdgcn_perm(f1, f0, 0x05040100u)), cap);
          const u16x2 m23 = __builtin_elementwise_min(__builtin_bit_cast(u16x2, __builtin_amdgcn_perm(f3, f2, 0x05040100u)), cap);
          // (every byte even: the shift moves no bit across bytes)
          uint32_t word = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, m23), __builtin_bit_cast(uint32_t, m01), 0x06040200u) >> 1;
          const int b = pt * NWP + b0 + j;
          if (PAD) {
            // padding keys (j >= n) at level 127 with the capped ones
            const int real = n - (g * KG + 4 * b);
            word |= real >= 4 ? 0u : (real <= 0 ? 0x7f7f7f7fu : (0x7f7f7f7fu << (8 * real)));
          }
          P[b] = word;
        }
      }
    }
  }
  __syncthreads();  // every wave is done with the key operands
  issue_round(0);
  issue_round(1);

  // ---- 2. threshold: smallest tau with C(tau) >= keep, C(t) = #{h <= t}, by probes
  // next to the guess and bisection (as at d = 64) over levels below `top`, where
  // C(top) = every byte of the row is known to reach keep
  int tau = 0, less = 0, cl_lo = 0, cl_hi = 0;
  auto search = [&](int top) {
    const int tq = min(max(a.t0, 1), top - 1);
    int lo, hi, clo, llo, lhi, sl, sh;
    {
      const int sm = (int)lane_sad<NW>(P, (uint32_t)tq - 1u);
      const int s0 = (int)lane_sad<NW>(P, (uint32_t)tq);
      const int sp = (int)lane_sad<NW>(P, (uint32_t)tq + 1u);
      const int cx = (s0 - sm + 4 * NW) >> 1, cy = (sp - s0 + 4 * NW) >> 1;
      const int both = quad_rows_sum((cy << 16) | cx);
      const int ta = both & 0xffff, tb = both >> 16;
      const bool below = ta >= keep;
      const bool at = !below && tb >= keep;
      lo = below ? -1 : (at ? tq - 1 : tq);
      hi = below ? tq - 1 : (at ? tq : top);
      clo = below ? 0 : (at ? ta : tb);
      llo = below ? 0 : (at ? cx : cy);
      lhi = below ? cx : (at ? cy : 0);
      sl = sp;
      sh = sm;
    }
    while (__builtin_amdgcn_ballot_w64(hi - lo > 1) != 0) {
      const bool open = hi - lo > 1;
      int mid = hi == top ? lo + 1 : (lo == -1 ? hi - 1 : (lo + hi) >> 1);
      mid = open ? mid : hi;
      const bool next_lo = mid == lo + 1 && lo >= 0;
      const bool next_hi = mid == hi - 1 && hi < top && !next_lo;
      const int s1 = (int)lane_sad<NW>(P, (uint32_t)(next_lo ? mid + 1 : mid));
      int smid = next_lo ? sl : s1, snext = next_lo ? s1 : sh;
      if (__builtin_amdgcn_ballot_w64(open && !next_lo && !next_hi) != 0) {
        const int s2 = (int)lane_sad<NW>(P, (uint32_t)mid + 1u);
        snext = (next_lo || next_hi) ? snext : s2;
      }
      const int cm = (snext - smid + 4 * NW) >> 1;
      const int tm = quad_rows_sum(cm);
      const bool up = open && tm >= keep;
      const bool dn = open && tm < keep;
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
  };
  bool exact = false;  // wave-uniform: a row of this tile keeps keys at a capped level
  if (have) {
    search(127);
    exact = __builtin_amdgcn_ballot_w64(tau >= 127) != 0;
  }
  if (exact) {
    // Levels 127 and 128 and the padding share byte 127.  Count this lane's keys at
    // level 127 from their codes, then settle tau at 127 or 128 for the rows that
    // reached it (their C(126) < keep); rows with tau <= 126 keep it.
    int c127 = 0;
#pragma unroll
    for (int b = 0; b < NW; ++b) {
      const uint32_t x = P[b] ^ 0x7f7f7f7fu;
      const uint32_t z = ~(((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x | 0x7f7f7f7fu);  // bit 7: byte == 127
      if (z != 0u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = g * KG + 4 * b + e;
          if (((z >> (8 * e + 7)) & 1u) && j < n) {
            const uint4 c = kb[j];
            const int h = __builtin_popcount(q.x ^ c.x) + __builtin_popcount(q.y ^ c.y) +
                          __builtin_popcount(q.z ^ c.z) + __builtin_popcount(q.w ^ c.w);
            c127 += h == 127 ? 1 : 0;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int c127r = quad_rows_sum(c127);
    if (tau >= 127) {
      // (here less = C(126) and cl_lo = this lane's keys below 127; the search never
      // counted level 127, its upper bound from the start)
      const int pad = min(max((g + 1) * KG - max(n, g * KG), 0), KG);  // this lane's padding keys
      if (less + c127r >= keep) {
        tau = 127;
        cl_hi = cl_lo + c127;
      } else {
        tau = 128;
        less += c127r;
        const int c128 = KG - cl_lo - c127 - pad;
        cl_lo += c127;
        cl_hi = cl_lo + c128;
      }
    }
  }
  // ---- the rows of rounds 0 and 1 are in place
  wait_vmem();
  __syncthreads();

  // ---- 3. ties
  const int ceq = cl_hi - cl_lo;
  const int before = quad_rows_excl(ceq, g);
  const int take = min(max(keep - less - before, 0), ceq);
  const uint32_t kidx = byte_bcast((uint32_t)(127 - tau));
  const uint32_t ktau = byte_bcast((uint32_t)tau);
  const uint32_t kcut = 127u - (uint32_t)take;

  // ---- 4-5. weights and A*V, two passes of 64 channels
  const bf16x8 ones = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(lds_u8*)one_pairs);
  const uint32_t vrow0 = (uint32_t)(g * KR + (r >> 2));
  const uint32_t vsw = vswz((uint32_t)g, vrow0);
  uint32_t voff[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) voff[tt] = vrow0 * 128u + 32u * ((uint32_t)tt ^ vsw) + 8u * (uint32_t)(r & 3);
  auto loadB = [&](int rg, int cl, bf16x8 (&Bv)[4]) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      lds_u8* const ad = vbuf(rg) + voff[tt] + 8 * cl * 128;
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ad);
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ad + 4 * 128));
      Bv[tt] = __builtin_bit_cast(bf16x8, i16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
    }
  };
  auto output = [&](int pass, const f32x4 (&acc)[4], const f32x4& accz) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = t * 16 + 4 * g + e;
      const float inv = __builtin_amdgcn_rcpf(accz[e]);  // (Z >= 1: the weight at tau is 1)
      if (row < n) {
        float* o = a.out + (hb + row) * kD2 + 64 * pass + r;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) o[16 * tt] = acc[tt][e] * inv;
      }
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
  auto run_av = [&]() {
    f32x4 acc[4], accz;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accz = f32x4{0.f, 0.f, 0.f, 0.f};
    int run = 0;  // keys at tau met so far in this lane (ascending j)
    int32_t* idst = nullptr;
    int ipos = 0;
    if (IDX) {
      ipos = quad_rows_excl(cl_lo + take, g);
      idst = a.idx + (hb + (i < n ? i : 0)) * (size_t)keep;
    }
    // step c of the lane's keys g KG + 8 c + 0..7: the tie cut and the table entries
    // per-pass copies of the tie constants, opaque to the compiler: the second pass
    // redoes the tie cut instead of keeping the first pass's words for every step
    uint32_t pk_idx = kidx, pk_tau = ktau, pk_cut = kcut;
    auto prep = [&](int c, bool list, uint32_t (&ent)[8]) {
      const uint32_t P0 = P[2 * c], P1 = P[2 * c + 1];
      const uint32_t E0 = ~xor_add(P0, pk_tau, 0x7f7f7f7fu) & kM;
      const uint32_t E1 = ~xor_add(P1, pk_tau, 0x7f7f7f7fu) & kM;
      const int mid = __builtin_popcount(E0) + run;
      const int run1 = __builtin_popcount(E1) + mid;
      const bool over = run1 > take;
      uint32_t U0 = over ? E0 : 0u, U1 = over ? E1 : 0u;
      if (over && !(run >= take)) {
        U0 = E0 & byte_prefix((E0 >> 7) + pk_cut + (uint32_t)run);
        U1 = E1 & byte_prefix((E1 >> 7) + pk_cut + (uint32_t)mid);
      }
      run = run1;
      // h - tau + 127 per byte, plus 128 for a key at tau that is not taken
      const uint32_t I0 = P0 + pk_idx + U0, I1 = P1 + pk_idx + U1;
      if (IDX && list && i < n) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint32_t ib = ((b < 4 ? I0 : I1) >> (8 * (b & 3))) & 0xffu;
          if (ib <= 127u && ipos < keep) idst[ipos++] = g * KG + 8 * c + b;
        }
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        ent[b] = tab[(I0 >> (8 * b)) & 0xffu];
        ent[4 + b] = tab[(I1 >> (8 * b)) & 0xffu];
      }
    };
    // the passes as a loop (the rounds of a pass unrolled, so that the words of P and
    // the buffer of each round are fixed at compile time)
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      asm volatile("" : "+v"(pk_idx), "+v"(pk_tau), "+v"(pk_cut));
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int rg = pass * R + rr;
        const int par = R % 2 == 0 ? rr : rg;  // the round's buffer parity
        if (rg > 0) {
          wait_vmem();
          __syncthreads();
          if (rg + 1 < 2 * R) issue_round(rg + 1);
        }
        if (rg * 4 / (2 * R) == 1 && (rg - 1) * 4 / (2 * R) != 1) __builtin_amdgcn_s_setprio(2);
        if (rg * 4 / (2 * R) == 2 && (rg - 1) * 4 / (2 * R) != 2) __builtin_amdgcn_s_setprio(1);
        if (rg * 4 / (2 * R) == 3 && (rg - 1) * 4 / (2 * R) != 3) __builtin_amdgcn_s_setprio(0);
        if (have) {
          bf16x8 Bv[2][4];
          uint32_t ent[2][8];
          loadB(par, 0, Bv[0]);
          prep(rr * NKR, pass == 0, ent[0]);
#pragma unroll
          for (int cl = 0; cl < NKR; ++cl) {
            bf16x8 A_hi, A_lo;
            make_a(ent[cl & 1], A_hi, A_lo);
            if (cl + 1 < NKR) prep(rr * NKR + cl + 1, pass == 0, ent[(cl + 1) & 1]);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, Bv[cl & 1][tt], acc[tt], 0, 0, 0);
            if (pass == 0) accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, ones, accz, 0, 0, 0);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
              acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, Bv[cl & 1][tt], acc[tt], 0, 0, 0);
            if (pass == 0) accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, ones, accz, 0, 0, 0);
            if (cl + 1 < NKR) loadB(par, cl + 1, Bv[(cl + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if (pass == 0 && have) {
        // channels 0..63 done: write them, keep Z, start the second pass
        output(0, acc, accz);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        run = 0;
      }
    }
    if (have) output(1, acc, accz);
  };
  // The exact path: every key's level again from its code (no distance words, so the
  // loops stay rolled and the registers those of the fast path), the same rounds and
  // barriers as the fast path.
  auto run_av_exact = [&]() {
    f32x4 acc[4], accz;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accz = f32x4{0.f, 0.f, 0.f, 0.f};
    int run = 0;
    int32_t* idst = nullptr;
    int ipos = 0;
    if (IDX) {
      ipos = quad_rows_excl(cl_lo + take, g);
      idst = a.idx + (hb + (i < n ? i : 0)) * (size_t)keep;
    }
#pragma unroll 1
    for (int rg = 0; rg < 2 * R; ++rg) {
      const int pass = rg >= R ? 1 : 0;
      const int rr = rg - pass * R;
      if (rg > 0) {
        wait_vmem();
        __syncthreads();
        if (rg + 1 < 2 * R) issue_round(rg + 1);
      }
      if (rg == R) {
        output(0, acc, accz);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        run = 0;
      }
#pragma unroll 1
      for (int cl = 0; cl < NKR; ++cl) {
        const int c = rr * NKR + cl;
        uint32_t ent[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int j = g * KG + 8 * c + b;
          int h = 255;  // padding keys: never kept
          if (j < n) {
            const uint4 cc = kb[j];
            h = __builtin_popcount(q.x ^ cc.x) + __builtin_popcount(q.y ^ cc.y) + __builtin_popcount(q.z ^ cc.z) +
                __builtin_popcount(q.w ^ cc.w);
          }
          const bool kept = h < tau || (h == tau && run < take);
          run += h == tau ? 1 : 0;
          ent[b] = kept ? tabg[tau - h] : 0u;
          if (IDX && pass == 0 && kept && i < n && ipos < keep) idst[ipos++] = j;
        }
        bf16x8 Bv[4], A_hi, A_lo;
        loadB(rg, cl, Bv);
        make_a(ent, A_hi, A_lo);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, Bv[tt], acc[tt], 0, 0, 0);
        if (pass == 0) accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, ones, accz, 0, 0, 0);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, Bv[tt], acc[tt], 0, 0, 0);
        if (pass == 0) accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, ones, accz, 0, 0, 0);
      }
    }
    output(1, acc, accz);
  };
  if (exact)
    run_av_exact();
  else
    run_av();
}

template <int NK, bool PAD, bool IDX>
hipError_t launch_d128_nk(const MfmaKArgs& ka, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((topn_mfma_d128_kernel<NK, PAD, IDX>), grid, block, 0, s, ka);
  return hipGetLastError();
}

template <int NK>
hipError_t launch_d128_pad(const MfmaKArgs& ka, bool pad, dim3 grid, dim3 block, hipStream_t s) {
  if (ka.idx != nullptr)
    return pad ? launch_d128_nk<NK, true, true>(ka, grid, block, s) : launch_d128_nk<NK, false, true>(ka, grid, block, s);
  return pad ? launch_d128_nk<NK, true, false>(ka, grid, block, s) : launch_d128_nk<NK, false, false>(ka, grid, block, s);
}

template <int NK, bool PAD, bool IDX, bool FK>
hipError_t launch_nk(const MfmaKArgs& ka, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((topn_mfma_kernel<NK, PAD, IDX, FK>), grid, block, 0, s, ka);
  return hipGetLastError();
}

template <int NK, bool FK>
hipError_t launch_pad(const MfmaKArgs& ka, bool pad, dim3 grid, dim3 block, hipStream_t s) {
  if (ka.idx != nullptr)
    return pad ? launch_nk<NK, true, true, FK>(ka, grid, block, s) : launch_nk<NK, false, true, FK>(ka, grid, block, s);
  return pad ? launch_nk<NK, true, false, FK>(ka, grid, block, s) : launch_nk<NK, false, false, FK>(ka, grid, block, s);
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
  const bool base = p.v_kind == 1 && p.alpha_q == nullptr && p.alpha_k == nullptr && p.brow == nullptr && p.n >= 1;
  if (p.d == kD2) return base && p.bias == nullptr && p.n <= 1024;
  if (p.d != kD) return false;
  if (p.bias == nullptr) return base && p.n <= 1024;
  return base && p.n <= 256;  // float keys: the heads whose table passes the level test
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
  ka.bias = p.bias;
  ka.H = (int)p.H;
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  const int64_t BH = p.B * p.H;
  ka.split = (ka.tiles + kWaves - 1) / kWaves;
  if (BH * ka.split >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(BH * ka.split));
  const dim3 block((unsigned)(64 * kWaves));
  const bool pad = p.n != 32 * NK;
  if (p.d == kD2) {
    switch (NK) {
      case 2: return launch_d128_pad<2>(ka, pad, grid, block, s);
      case 4: return launch_d128_pad<4>(ka, pad, grid, block, s);
      case 8: return launch_d128_pad<8>(ka, pad, grid, block, s);
      case 16: return launch_d128_pad<16>(ka, pad, grid, block, s);
      default: return launch_d128_pad<32>(ka, pad, grid, block, s);
    }
  }
  if (p.bias != nullptr) {
    switch (NK) {
      case 2: return launch_pad<2, true>(ka, pad, grid, block, s);
      case 4: return launch_pad<4, true>(ka, pad, grid, block, s);
      default: return launch_pad<8, true>(ka, pad, grid, block, s);
    }
  }
  switch (NK) {
    case 2: return launch_pad<2, false>(ka, pad, grid, block, s);
    case 4: return launch_pad<4, false>(ka, pad, grid, block, s);
    case 8: return launch_pad<8, false>(ka, pad, grid, block, s);
    case 16: return launch_pad<16, false>(ka, pad, grid, block, s);
    default: return launch_pad<32, false>(ka, pad, grid, block, s);
  }
}

}  // namespace had
