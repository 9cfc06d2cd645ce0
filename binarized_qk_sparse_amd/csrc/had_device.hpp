// Device-side helpers shared by the gfx950 kernels (wave64 primitives).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define HAD_DEVICE __device__ __forceinline__

namespace had {

constexpr int kWave = 64;

HAD_DEVICE int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Rank of this lane among the set lanes of `mask` below it.
HAD_DEVICE uint32_t mask_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

HAD_DEVICE uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

template <typename T>
HAD_DEVICE T uniform(T v) {
  return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// DPP controls (GFX9 encoding).
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

template <int CTRL>
HAD_DEVICE int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
HAD_DEVICE float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, false));
}

// Full-wave reductions on the DPP network: quad swaps, row rotations, then the
// row broadcasts carry the partial sums up to lane 63.  Result is wave-uniform.
constexpr int kQuadSwap1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int CTRL, int ROWMASK>
HAD_DEVICE int dppm_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xf, false);
}

HAD_DEVICE int wave_sum_i32(int v) {
  v += dpp_i<kQuadSwap1>(v);
  v += dpp_i<kQuadSwap2>(v);
  v += dpp_i<kRowRor4>(v);
  v += dpp_i<kRowRor8>(v);
  v += dppm_i<kRowBcast15, 0xa>(v);
  v += dppm_i<kRowBcast31, 0xc>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

HAD_DEVICE float as_f(int v) { return __builtin_bit_cast(float, v); }
HAD_DEVICE int as_i(float v) { return __builtin_bit_cast(int, v); }

HAD_DEVICE float wave_sum_f32(float v) {
  v += dpp_f<kQuadSwap1>(v);
  v += dpp_f<kQuadSwap2>(v);
  v += dpp_f<kRowRor4>(v);
  v += dpp_f<kRowRor8>(v);
  v += as_f(dppm_i<kRowBcast15, 0xa>(as_i(v)));
  v += as_f(dppm_i<kRowBcast31, 0xc>(as_i(v)));
  return as_f(__builtin_amdgcn_readlane(as_i(v), 63));
}

// Max over the wave (the masked-off rows of the broadcasts see -inf).
HAD_DEVICE float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f<kQuadSwap1>(v));
  v = fmaxf(v, dpp_f<kQuadSwap2>(v));
  v = fmaxf(v, dpp_f<kRowRor4>(v));
  v = fmaxf(v, dpp_f<kRowRor8>(v));
  v = fmaxf(v, as_f(__builtin_amdgcn_update_dpp(as_i(-INFINITY), as_i(v), kRowBcast15, 0xa, 0xf, false)));
  v = fmaxf(v, as_f(__builtin_amdgcn_update_dpp(as_i(-INFINITY), as_i(v), kRowBcast31, 0xc, 0xf, false)));
  return as_f(__builtin_amdgcn_readlane(as_i(v), 63));
}

HAD_DEVICE uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)dpp_i<kQuadSwap1>((int)v));
  v = min(v, (uint32_t)dpp_i<kQuadSwap2>((int)v));
  v = min(v, (uint32_t)dpp_i<kRowRor4>((int)v));
  v = min(v, (uint32_t)dpp_i<kRowRor8>((int)v));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kRowBcast15, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, kRowBcast31, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

HAD_DEVICE uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<kQuadSwap1>((int)v));
  v = max(v, (uint32_t)dpp_i<kQuadSwap2>((int)v));
  v = max(v, (uint32_t)dpp_i<kRowRor4>((int)v));
  v = max(v, (uint32_t)dpp_i<kRowRor8>((int)v));
  v = max(v, (uint32_t)dppm_i<kRowBcast15, 0xa>((int)v));
  v = max(v, (uint32_t)dppm_i<kRowBcast31, 0xc>((int)v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Exclusive prefix sum over the 64 lanes on the DPP network (lane 0 gets 0).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

HAD_DEVICE int wave_excl_scan_i32(int v) {
  int x = v;
  x += dpp_i<kRowShr1>(x);  // lanes shifted in from outside the row read 0
  x += dpp_i<kRowShr2>(x);
  x += dpp_i<kRowShr4>(x);
  x += dpp_i<kRowShr8>(x);
  x += dppm_i<kRowBcast15, 0xa>(x);
  x += dppm_i<kRowBcast31, 0xc>(x);
  return x - v;
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Two floats -> packed fp16 (round to nearest even).
HAD_DEVICE uint32_t pack_half2(float lo, float hi) {
  const half2v h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// bf16 bits -> float (exact widening).
HAD_DEVICE float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
HAD_DEVICE float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Order-preserving map float -> uint32 (a larger float maps to a larger key).
HAD_DEVICE uint32_t ordered_key(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
HAD_DEVICE float from_ordered_key(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, b);
}

// The rr-th largest (1-based) of the values x held by lanes [0, cnt) of the wave
// (1 <= rr <= cnt <= 64), by quickselect: each round compares every live value
// with a pivot read from one live lane and keeps the side that holds the rank.
// A round removes at least the pivot, so at most cnt rounds run; the pivot lane
// is the first live one at or after a start position that moves every round, so
// values in lane order do not make every round remove only one value.
HAD_DEVICE uint32_t wave_select_desc(uint32_t x, int cnt, int rr) {
  uint64_t live = cnt >= 64 ? ~0ull : ((1ull << cnt) - 1ull);
  int rem = rr;
  uint32_t start = 0;
  for (;;) {
    const uint64_t from = live & (~0ull << start);
    const int p = (int)__builtin_ctzll(from != 0 ? from : live);
    const uint32_t pv = (uint32_t)__builtin_amdgcn_readlane((int)x, p);
    const uint64_t gt = ballot(x > pv) & live;
    const int g = __builtin_popcountll(gt);
    if (g >= rem) {
      live = gt;
    } else {
      const uint64_t eq = ballot(x == pv) & live;
      const int e = __builtin_popcountll(eq);
      if (g + e >= rem) return pv;
      rem -= g + e;
      live &= ~(gt | eq);
    }
    start = (start + 23u) & 63u;
  }
}

// Per-channel integer code of x at scale s (inv = v_rcp_f32(s)) with L levels
// each side of zero (127: int8; 7: 4-bit V): clamp(rint(fl(x / s)), -L, L) as a
// byte, 0 when s is 0.  x * (1/s) is within 2 ulp of the correctly rounded
// quotient fl(x / s), i.e. within 2^-16 for |x / s| <= 128, so the two can round
// to different integers only when the quotient lies near a tie k + 1/2; there
// the exact division decides (as it does for a denormal scale, whose reciprocal
// is not representable).
template <int L = 127>
HAD_DEVICE uint32_t quant_i8(float x, float s, float inv) {
  if (!(s > 0.0f)) return 0u;
  float y = x * inv;
  if (s < 0x1p-125f || fabsf(y - floorf(y) - 0.5f) < 0x1p-12f) y = __fdiv_rn(x, s);
  float r = rintf(y);
  r = fminf(fmaxf(r, -(float)L), (float)L);
  return (uint32_t)((int32_t)r) & 0xffu;
}

// ---- two-dimensional decomposable bias (row + column offset tables, class token)
// Position code of token t: bit 31 marks the class token, bits 16..30 hold the
// grid row and bits 0..15 the column (both 0 for the class token, so every
// table index below stays in range).
HAD_DEVICE uint32_t grid_pos(int t, int gw, int cls) {
  if (t < cls) return 0x80000000u;
  const int p = t - cls;
  const int r = p / gw;
  return ((uint32_t)r << 16) | (uint32_t)(p - r * gw);
}

// The tables of head h, [rows 2gh-1 | columns 2gw-1 | class->patch, patch->class,
// class->class], into tab[0 .. bias2d floats) (threads tid, tid + nt, ...).
HAD_DEVICE void stage_bias2d(float* tab, const float* R, const float* C, const float* X, int h, int gh, int gw,
                             int tid, int nt) {
  const int nr = 2 * gh - 1, nc = 2 * gw - 1;
  for (int k = tid; k < nr + nc + 3; k += nt)
    tab[k] = k < nr ? R[(size_t)h * nr + k]
                    : (k < nr + nc ? C[(size_t)h * nc + (k - nr)] : (X != nullptr ? X[h * 3 + (k - nr - nc)] : 0.0f));
}

// Bias of the pair (query at qpos, key at kpos): R[rj - ri + gh - 1] + C[cj - ci + gw - 1]
// (rounded once) between patches, a class value when either is the class token.
HAD_DEVICE float bias2d_pair(const float* tab, int gh, int gw, uint32_t qpos, uint32_t kpos) {
  const int ri = (int)((qpos >> 16) & 0x7fffu), ci = (int)(qpos & 0xffffu);
  const int rj = (int)((kpos >> 16) & 0x7fffu), cj = (int)(kpos & 0xffffu);
  const float pp = __fadd_rn(tab[rj - ri + gh - 1], tab[(2 * gh - 1) + cj - ci + gw - 1]);
  const float* X = tab + (2 * gh - 1) + (2 * gw - 1);
  const bool qc = (qpos >> 31) != 0, kc = (kpos >> 31) != 0;
  return qc ? (kc ? X[2] : X[0]) : (kc ? X[1] : pp);
}

// Canonical float32 logit: each operation rounded as written, no contraction.
HAD_DEVICE float canonical_logit(float aq, float ak, int dot, float inv_sqrt_d, float bias) {
  float t = __fmul_rn(aq, ak);
  float u = __fmul_rn(t, (float)dot);
  float v = __fmul_rn(u, inv_sqrt_d);
  return __fadd_rn(v, bias);
}

// The packed code of one token for head_dim D: D / 32 words, bit c % 32 of word
// c / 32 set for a -1 code (the layout had_pack writes).
template <int D>
struct Code {
  uint32_t w[D / 32];
};

template <int D>
HAD_DEVICE Code<D> load_code(const uint32_t* base, size_t row) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  Code<D> c;
  if constexpr (D == 64) {
    const uint2 v = reinterpret_cast<const uint2*>(base)[row];
    c.w[0] = v.x;
    c.w[1] = v.y;
  } else {
    const uint4 v = reinterpret_cast<const uint4*>(base)[row];
    c.w[0] = v.x;
    c.w[1] = v.y;
    c.w[2] = v.z;
    c.w[3] = v.w;
  }
  return c;
}

// Hamming distance of two codes.
template <int D>
HAD_DEVICE int hamming(const Code<D>& x, const Code<D>& y) {
  int h = 0;
#pragma unroll
  for (int w = 0; w < D / 32; ++w) h = __builtin_popcount(x.w[w] ^ y.w[w]) + h;
  return h;
}

// XCD-aware remap of the linear workgroup id: consecutive logical ids land on
// the same XCD (hardware dispatches workgroup w to XCD w % 8), so the blocks
// that share a head's keys and values share one L2.
HAD_DEVICE uint32_t xcd_remap(uint32_t w, uint32_t nwg) {
  constexpr uint32_t kXcd = 8;
  uint32_t per = nwg / kXcd;
  uint32_t full = per * kXcd;
  if (w >= full) return w;  // the remainder keeps its id
  return (w % kXcd) * per + (w / kXcd);
}

}  // namespace had
