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

// The values of this lane and of lane l ^ OFF (OFF = 4, 8, 16 or 32), on the VALU
// where the hardware has the exchange: a DPP rotation by 8 within each 16-lane row
// (lane l meets l ^ 8), the gfx950 permlane swaps across 16-lane rows and 32-lane
// halves (which hand both lanes the pair in the same order); a bpermute for 4.  The
// two values may come in either order, so a commutative combination of them gives
// both lanes the same bits.
template <int OFF>
HAD_DEVICE void xor_pair(uint32_t x, uint32_t& a, uint32_t& b) {
  static_assert(OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "lane distance");
  if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  } else if constexpr (OFF == 8) {
    a = x;
    b = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, true);  // row_ror:8
  } else {
    a = x;
    b = (uint32_t)__shfl_xor((int)x, OFF, 64);
  }
}

// Butterfly over the lanes OFF, 2 OFF, .., 32 apart: f(this lane's value, the other's)
// at each step, f commutative (float64 sum, float max), so every lane ends with the
// same bits.
template <int OFF, class F>
HAD_DEVICE double butterfly_f64(double v, F f) {
  if constexpr (OFF >= 64) {
    return v;
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    uint32_t al, bl, ah, bh;
    xor_pair<OFF>((uint32_t)u, al, bl);
    xor_pair<OFF>((uint32_t)(u >> 32), ah, bh);
    const double a = __builtin_bit_cast(double, ((uint64_t)ah << 32) | al);
    const double b = __builtin_bit_cast(double, ((uint64_t)bh << 32) | bl);
    return butterfly_f64<2 * OFF>(f(a, b), f);
  }
}
template <int OFF, class F>
HAD_DEVICE float butterfly_f32(float v, F f) {
  if constexpr (OFF >= 64) {
    return v;
  } else {
    uint32_t a, b;
    xor_pair<OFF>(__builtin_bit_cast(uint32_t, v), a, b);
    return butterfly_f32<2 * OFF>(f(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)), f);
  }
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

// x / 255 rounded to nearest even, as __fdiv_rn(x, 255.0f) gives it, in three
// operations: q0 = fl(x * y) with y = fl(1 / 255), the exact remainder
// r = fma(-q0, 255, x), and q = fma(r, y, q0).  Checked against IEEE division for
// every finite float, denormals included (the identity holds for this divisor; it
// is not a general division).
HAD_DEVICE float div255_rn(float x) {
  constexpr float y = 1.0f / 255.0f;
  const float q0 = __fmul_rn(x, y);
  const float r = __builtin_fmaf(-q0, 255.0f, x);
  return __builtin_fmaf(r, y, q0);
}

// Channel c (0..7) of a word of eight 4-bit two's-complement codes (nibble c),
// sign-extended.
HAD_DEVICE int nibble_s4(uint32_t w, int c) { return (int)(w << (28 - 4 * c)) >> 28; }

// ---- two-dimensional decomposable bias (row + column offset tables, class token)
// The tables are staged with the class token's values folded in, so that every
// pair costs two table reads and one addition whatever its kind:
//   row part  R': [0, 2gh-1) R; with a class token also [2gh-1, 3gh-1) patch->class,
//                 [3gh-1, 4gh-1) class->patch, and 5gh-2 class->class;
//   column part C' (after R'): [0, 2gw-1) C, zeros elsewhere (5gw-1 entries with a
//                 class token).
// Key code: (kr << 16) | kc, with (rj, cj) for a patch and (2gh-1, 2gw-1) for the
// class token; query bases: (gh-1-ri, gw-1-ci) for a patch and (3gh-1, 3gw-1) for
// the class token.  B = R'[kr + qr] + C'[kc + qc]: for two patches that is
// R[rj - ri + gh - 1] + C[cj - ci + gw - 1], and a class-token pair adds 0 to its
// value.
HAD_DEVICE int bias2d_rows(int gh, int cls) { return cls ? 5 * gh - 1 : 2 * gh - 1; }
HAD_DEVICE int bias2d_cols(int gw, int cls) { return cls ? 5 * gw - 1 : 2 * gw - 1; }

HAD_DEVICE void stage_bias2d(float* tab, const float* R, const float* C, const float* X, int h, int gh, int gw,
                             int cls, int tid, int nt) {
  const int nr = bias2d_rows(gh, cls), nc = bias2d_cols(gw, cls);
  for (int k = tid; k < nr + nc; k += nt) {
    float v = 0.0f;
    if (k < nr) {
      if (k < 2 * gh - 1) v = R[(size_t)h * (2 * gh - 1) + k];
      else if (k < 3 * gh - 1) v = X[h * 3 + 1];
      else if (k < 4 * gh - 1) v = X[h * 3 + 0];
      else if (k == 5 * gh - 2) v = X[h * 3 + 2];
    } else if (k - nr < 2 * gw - 1) {
      v = C[(size_t)h * (2 * gw - 1) + (k - nr)];
    }
    tab[k] = v;
  }
}

HAD_DEVICE uint32_t bias2d_key(int t, int gh, int gw, int cls) {
  if (t < cls) return ((uint32_t)(2 * gh - 1) << 16) | (uint32_t)(2 * gw - 1);
  const int p = t - cls;
  const int r = p / gw;
  return ((uint32_t)r << 16) | (uint32_t)(p - r * gw);
}

// Query bases into the staged tables (the column base includes the row part's length).
HAD_DEVICE int2 bias2d_query(int i, int gh, int gw, int cls) {
  const int nr = bias2d_rows(gh, cls);
  if (i < cls) return make_int2(3 * gh - 1, nr + 3 * gw - 1);
  const int p = i - cls;
  const int r = p / gw;
  return make_int2(gh - 1 - r, nr + gw - 1 - (p - r * gw));
}

HAD_DEVICE float bias2d_lookup(const float* tab, int2 q, uint32_t key) {
  return __fadd_rn(tab[(int)(key >> 16) + q.x], tab[(int)(key & 0xffffu) + q.y]);
}

// Whether a head's relative-position table leaves the order of the logits of plain
// sign codes at head_dim 64 to their Hamming levels except within one level: its
// values (tmin .. tmax over all 2n - 1 entries, none NaN) span less than one logit
// step 2 / sqrt(64) = 0.25.  l = fl(v(h) + T) with v(h) = (64 - 2h) / 8 exact, so two
// keys at levels h < h' differ by at least 0.25 - (tmax - tmin) > 0.01 before
// rounding and by at most 2 * 2^-24 * 1008 through it (|T| <= 1000).
HAD_DEVICE bool bias_levels_separate(float tmin, float tmax, bool has_nan) {
  return !has_nan && tmax - tmin < 0.24f && tmax <= 1000.0f && tmin >= -1000.0f;
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

// d - 2 h for two codes: popcounts chained through the accumulate operand of
// v_bcnt_u32_b32 and one 24-bit multiply-add (the compiler would otherwise add
// the popcounts, shift and subtract).
template <int D>
HAD_DEVICE int code_dot(const Code<D>& x, const Code<D>& y) {
  uint32_t h;
  asm("v_bcnt_u32_b32 %0, %1, 0" : "=v"(h) : "v"(x.w[0] ^ y.w[0]));
#pragma unroll
  for (int w = 1; w < D / 32; ++w) asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(h) : "v"(x.w[w] ^ y.w[w]), "v"(h));
  int dot;
  asm("v_mad_i32_i24 %0, %1, -2, %2" : "=v"(dot) : "v"(h), "v"(D));
  return dot;
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
