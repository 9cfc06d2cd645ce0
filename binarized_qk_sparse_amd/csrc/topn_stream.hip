// Top-N binarized attention for long sequences (n above what one workgroup can
// hold on chip), one wavefront per query.
//
// Same method and arithmetic as the resident kernel (Hamming Attention
// Distillation summary: per-query top-N; BinaryAttention sections 2.2-2.4:
// scaled codes, bias, quantized A*V).  Differences:
//  * keys stream through LDS in chunks of 128 keys per wave (codes, alpha_k and the
//    bias offsets the workgroup's queries touch), shared by the workgroup's
//    waves, which process one query each in lockstep over the chunks;
//  * the top-N is streaming: a per-wave candidate buffer in LDS admits keys
//    whose logit beats the current threshold; when it fills, an interpolation
//    search finds a value with between N and N + 128 entries at or above it,
//    which becomes the threshold (an exact selection, ties to the lower key
//    index, when heavy ties defeat the search), and the exact selection runs
//    once more at the end.  Keys arrive in ascending j, so a later key with a
//    logit equal to the threshold can never displace a kept one, and the buffer
//    stays in ascending key order;
//  * V (or int8 V) rows are gathered from global memory (L2), eight lanes per
//    kept key.
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

// head_dim D is 64 or 128 (codes of D / 32 words).  A workgroup of W waves
// (W = 8 or 16) streams keys in LDS chunks of 128 W.  Each wave's candidate buffer
// holds CAP entries: 768 (kept sets up to 704), or 1536 for larger kept sets (up to
// 1472; eight waves, one workgroup per CU).
constexpr int kCapSmall = 768;
constexpr int kCapBig = 1536;

struct StreamKArgs {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const float* aq;
  const float* ak;
  const float* bias;
  const void* v;
  const float* vscale;
  float* out;
  int32_t* idx;
  int H, n, keep, lcap, tiles;
  float isd;
  // two-dimensional decomposable bias in place of `bias` (brow != NULL)
  const float* brow;
  const float* bcol;
  const float* bcls;
  int gh, gw, cls;
};

// LDS layout (bytes) for head_dim D, W waves and CAP buffer entries per wave
template <int D, int W, int CAP = kCapSmall>
struct Lds {
  static constexpr int kChunk = 128 * W;                             // keys per chunk
  static constexpr uint32_t kCodeOff = 0;                           // Code<D>[kChunk]
  static constexpr uint32_t kAkOff = kCodeOff + kChunk * (D / 8);   // float[kChunk]
  static constexpr uint32_t kBiasOff = kAkOff + kChunk * 4;         // float[kChunk + W]
  static constexpr uint32_t kBufOff = kBiasOff + (kChunk + 64) * 4;  // uint2[W][CAP]
  static constexpr uint32_t kCandOff = kBufOff + W * CAP * 8;       // uint2[W][64]
  static constexpr int kTab = W == 16 ? 1536 : 512;                  // floats of two-dimensional bias tables
  static constexpr uint32_t kTabOff = kCandOff + W * 64 * 8;         // float[kTab]
  static constexpr uint32_t kTotal = kTabOff + kTab * 4;
};
static_assert(Lds<128, 16>::kTotal <= 160 * 1024, "LDS");
static_assert(2 * Lds<128, 8>::kTotal <= 160 * 1024, "LDS: two workgroups of eight waves per CU");
static_assert(Lds<128, 8, kCapBig>::kTotal <= 160 * 1024, "LDS: one workgroup of eight waves per CU");

// Byte transpose of four words: byte k of out[m] is byte m of in[k].
HAD_DEVICE void transpose_bytes4(const uint32_t (&in)[4], uint32_t (&out)[4]) {
  const uint32_t lo01 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // in0.b0 in1.b0 in0.b1 in1.b1
  const uint32_t hi01 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // in0.b2 in1.b2 in0.b3 in1.b3
  const uint32_t lo23 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

template <int VK, int D>
constexpr int row_bytes() {
  return VK == 0 ? D * 4 : (VK == 1 ? D * 2 : (VK == 2 ? D : D / 2));
}

// Exact top-`keep` of the first `cnt` buffer entries (entry order = key order),
// ties to the earlier entry.  Rewrites the buffer with the kept entries in
// order and returns their count (min(cnt, keep)); `vstar` receives the value
// of the worst kept entry and `lmax` the best.
template <int CAP>
HAD_DEVICE int select_compact(uint2* buf, uint2* cand, int cnt, int keep, int lane, float* vstar_out,
                              float* lmax_out) {
  constexpr int kR = CAP / 64;
  float vals[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int e = lane + 64 * r;
    vals[r] = e < cnt ? __builtin_bit_cast(float, buf[e].x) : -INFINITY;
  }
  float lmax = -INFINITY, lmin = INFINITY;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    lmax = fmaxf(lmax, vals[r]);
    lmin = fminf(lmin, vals[r] == -INFINITY ? INFINITY : vals[r]);
  }
  lmax = wave_max_f32(lmax);
  lmin = -wave_max_f32(-lmin);
  *lmax_out = lmax;
  auto count_ge = [&](float t) {
    int c = 0;
#pragma unroll
    for (int r = 0; r < kR; ++r) c += __builtin_popcountll(ballot(vals[r] >= t));
    return c;
  };
  if (cnt <= keep) {
    *vstar_out = lmin;
    return cnt;
  }
  float vstar;
  int need;
  const int ctop = count_ge(lmax);
  if (ctop >= keep) {
    vstar = lmax;
    need = keep;
  } else {
    float lo = lmin, hi = lmax;
    int clo = cnt, chi = ctop;
    bool split = true;
    while (clo - chi > 64) {
      const float mid = 0.5f * lo + 0.5f * hi;
      if (!(mid > lo && mid < hi)) {
        split = false;
        break;
      }
      const int cm = count_ge(mid);
      if (cm >= keep) {
        lo = mid;
        clo = cm;
      } else {
        hi = mid;
        chi = cm;
      }
    }
    if (!split) {
      vstar = lo;
      need = keep - chi;
    } else {
      int cb = 0;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const bool c = vals[r] >= lo && vals[r] < hi;
        const uint64_t m = ballot(c);
        const int pos = cb + (int)mask_rank(m);
        if (c && pos < 64) cand[pos] = make_uint2(ordered_key(vals[r]), 0u);
        cb += __builtin_popcountll(m);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const uint32_t ck = lane < cb ? cand[lane].x : 0u;
      const int rr = keep - chi;
      const uint32_t L = wave_select_desc(ck, cb, rr);  // lanes >= cb hold 0, below every key
      vstar = from_ordered_key(L);
      need = keep - chi - __builtin_popcountll(ballot(ck > L));
    }
  }
  // the need-th entry (in order) holding vstar
  int estar = INT_MAX, seen = 0;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const uint64_t Em = ballot(vals[r] == vstar);
    const int e = __builtin_popcountll(Em);
    if (estar == INT_MAX && seen + e >= need) {
      uint64_t x = Em;
      for (int k = 0; k < need - seen - 1; ++k) x &= x - 1;
      estar = 64 * r + (int)__builtin_ctzll(x);
    }
    seen += e;
  }
  // keep l > vstar, or l == vstar up to entry estar; rewrite in order
  uint2 ent[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int e = lane + 64 * r;
    ent[r] = e < cnt ? buf[e] : make_uint2(0u, 0u);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int base = 0;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int e = lane + 64 * r;
    const bool sel = vals[r] > vstar || (vals[r] == vstar && e <= estar);
    const uint64_t Sm = ballot(sel);
    if (sel) buf[base + (int)mask_rank(Sm)] = ent[r];
    base += __builtin_popcountll(Sm);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  *vstar_out = vstar;
  return base;
}

// Entries an intermediate compaction may keep above the top-`keep`.
constexpr int kSlack = 128;

template <int R>
HAD_DEVICE int count_ge_rows(const float (&v)[R], float t) {
  int c = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) c += __builtin_popcountll(ballot(v[r] >= t));
  return c;
}

// Sequences of at least this many keys start each row's stream from a threshold taken
// from the logits of its first chunk.
constexpr int kSampleMinN = 4096;

// A threshold t from R values per lane such that about m of the wave's values are
// >= t: an interpolation search between the extremes that stops once [m, m + m / 2 + 8]
// values are >= t, else returns the highest t tried with at least m values >= t (the
// minimum at worst).
template <int R>
HAD_DEVICE float sample_threshold(const float (&v)[R], int m) {
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    lo = fminf(lo, v[r]);
    hi = fmaxf(hi, v[r]);
  }
  lo = -wave_max_f32(-lo);  // count_ge(lo) = 64 R >= m
  hi = wave_max_f32(hi);
  int clo = 64 * R, chi = count_ge_rows(v, hi);
  if (chi >= m) return hi;
  const int top = m + m / 2 + 8;
  for (int it = 0; it < 10; ++it) {
    float f = (float)(clo - (m + top) / 2) / (float)(clo - chi);
    f = fminf(fmaxf(f, 0.0625f), 0.9375f);
    const float mid = lo + f * (hi - lo);
    if (!(mid > lo && mid < hi)) break;
    const int cm = count_ge_rows(v, mid);
    if (cm < m) {
      hi = mid;
      chi = cm;
    } else {
      lo = mid;
      clo = cm;
      if (cm <= top) break;
    }
  }
  return lo;
}

// Intermediate compaction, cheaper than the exact selection: finds a value t
// with keep <= #{l >= t} <= keep + kSlack by interpolation search between theta
// (every entry is above it) and the largest entry, keeps the entries with
// l >= t in order, raises theta to t and returns their count.  This drops no
// entry of the final selection: t is at most the keep-th largest value, and a
// later key with l <= t ranks below the keep kept entries at or above t (equal
// values go to the lower key index).  Returns -1 when no such t turns up within
// a few steps (heavy ties); the caller then runs the exact selection.
template <int CAP>
HAD_DEVICE int compact_approx(uint2* buf, int cnt, int keep, int lane, float* theta) {
  constexpr int kR = CAP / 64;
  uint2 ent[kR];
  float vals[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int e = lane + 64 * r;
    ent[r] = e < cnt ? buf[e] : make_uint2(0xff800000u, 0u);  // -inf: empty slot
    vals[r] = __builtin_bit_cast(float, ent[r].x);
  }
  float hi = -INFINITY;
#pragma unroll
  for (int r = 0; r < kR; ++r) hi = fmaxf(hi, vals[r]);
  hi = wave_max_f32(hi);
  float lo = *theta;
  if (lo == -INFINITY) {
    float m = INFINITY;
#pragma unroll
    for (int r = 0; r < kR; ++r) m = fminf(m, vals[r] == -INFINITY ? INFINITY : vals[r]);
    lo = -wave_max_f32(-m);  // the smallest entry: #{l >= lo} = cnt
  }
  int clo = cnt, chi = count_ge_rows(vals, hi);
  const int top = keep + kSlack;
  float t = hi;
  int ct = chi;
  if (chi < keep) {
    ct = -1;
    for (int it = 0; it < 8; ++it) {
      float f = (float)(clo - (keep + kSlack / 2)) / (float)(clo - chi);
      f = fminf(fmaxf(f, 0.125f), 0.875f);
      const float mid = lo + f * (hi - lo);
      if (!(mid > lo && mid < hi)) break;
      const int cm = count_ge_rows(vals, mid);
      if (cm < keep) {
        hi = mid;
        chi = cm;
      } else if (cm > top) {
        lo = mid;
        clo = cm;
      } else {
        t = mid;
        ct = cm;
        break;
      }
    }
  }
  if (ct < keep || ct > top) return -1;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int base = 0;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const bool sel = vals[r] >= t;
    const uint64_t Sm = ballot(sel);
    if (sel) buf[base + (int)mask_rank(Sm)] = ent[r];
    base += __builtin_popcountll(Sm);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  *theta = t;
  return base;
}

// eight fp32 channels of a row
struct F8 {
  float4 a, b;
};

template <typename T>
HAD_DEVICE T reduce_scatter8(T (&acc)[8], int k) {
  const bool u4 = k & 4, u2 = k & 2, u1 = k & 1;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const T snd = u4 ? acc[c] : acc[c + 4];
    const T kp = u4 ? acc[c + 4] : acc[c];
    acc[c] = kp + __shfl_xor(snd, 32, 64);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const T snd = u2 ? acc[c] : acc[c + 2];
    const T kp = u2 ? acc[c + 2] : acc[c];
    acc[c] = kp + __shfl_xor(snd, 16, 64);
  }
  const T snd = u1 ? acc[0] : acc[1];
  const T kp = u1 ? acc[1] : acc[0];
  return kp + __shfl_xor(snd, 8, 64);
}

// B2: the two-dimensional bias (a.brow != NULL), a separate instance so that the
// 1-D path carries none of its code
template <int VK, int D, int W, int CAP, bool B2>
__global__ __launch_bounds__(64 * W) void topn_stream_kernel(const StreamKArgs a) {
  // 64-key groups per block of the key loop: eight at head_dim 64, two at 128 (whose
  // codes take twice the registers and LDS reads per key)
  constexpr int kG = D == 64 ? 8 : 2;
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int ROWB = row_bytes<VK, D>();
  using L = Lds<D, W, CAP>;
  constexpr int kWaves = W;
  constexpr int kChunk = L::kChunk;
  Code<D>* codes = reinterpret_cast<Code<D>*>(smem + L::kCodeOff);
  float* aks = reinterpret_cast<float*>(smem + L::kAkOff);
  float* biasw = reinterpret_cast<float*>(smem + L::kBiasOff);  // 1-D: bias window; 2-D: key position codes
  float* tab = reinterpret_cast<float*>(smem + L::kTabOff);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint2* buf = reinterpret_cast<uint2*>(smem + L::kBufOff) + wave * CAP;
  uint2* cand = reinterpret_cast<uint2*>(smem + L::kCandOff) + wave * 64;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.tiles, tile = wg % a.tiles, hh = bh % a.H;
  const int n = a.n, keep = a.keep;
  const int i0 = tile * kWaves;  // one query per wave
  const int i = i0 + wave;
  const bool live = i < n;  // uniform per wave
  const int ic = live ? i : n - 1;
  const size_t row = (size_t)bh * n + ic;
  const Code<D> qq = load_code<D>(a.qbits, row);
  const float aqv = a.aq != nullptr ? a.aq[row] : 1.0f;
  constexpr bool b2 = B2;
  const int2 qb2 = b2 ? bias2d_query(ic, a.gh, a.gw, a.cls) : make_int2(0, 0);
  // two-dimensional bias: the head's tables, each entry + 0 (no -0, as for the 1-D
  // window below); the chunk loop's first barrier orders them before any use
  if (b2) {
    stage_bias2d(tab, a.brow, a.bcol, a.bcls, hh, a.gh, a.gw, a.cls, (int)threadIdx.x, (int)blockDim.x);
    for (int k = threadIdx.x; k < bias2d_floats(a.gh, a.gw, a.cls); k += blockDim.x) tab[k] = __fadd_rn(tab[k], 0.0f);
  }
  const size_t kb = (size_t)bh * n;  // first key row of the head
  const float* akg = a.ak != nullptr ? a.ak + (size_t)bh * n : nullptr;
  const int ilast = min(n, i0 + kWaves) - 1;

  // A chunk's key codes, alpha_k and bias window go global -> registers -> LDS;
  // the next chunk's loads are issued before the current chunk is processed, so
  // they land while it runs.  Bias offsets o = j - i + n - 1 for j in the chunk
  // and i in [i0, ilast]; zero without a table.  Adding +0 turns a -0 entry into
  // +0, so no logit v + b is ever -0 (an exact zero sum rounds to +0) and equal
  // logits have equal bits.
  constexpr int kPer = kChunk / (64 * kWaves);
  Code<D> pcode[kPer];
  float pak[kPer], pbias[kPer + 1];
  const float* biash = a.bias != nullptr ? a.bias + (size_t)hh * (2 * n - 1) : nullptr;
  auto fetch_chunk = [&](int c0) {
    const int cl = min(kChunk, n - c0);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kWaves;
      if (t < cl) {
        pcode[r] = load_code<D>(a.kbits, kb + c0 + t);
        pak[r] = akg != nullptr ? akg[c0 + t] : 1.0f;
      }
    }
    const int ob = c0 - ilast + n - 1;
    const int cntb = cl + (ilast - i0);
#pragma unroll
    for (int r = 0; r <= kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kWaves;
      if (t < cntb) pbias[r] = biash != nullptr ? biash[ob + t] : 0.0f;
    }
  };
  auto store_chunk = [&](int c0) {
    const int cl = min(kChunk, n - c0);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kWaves;
      if (t < cl) {
        codes[t] = pcode[r];
        aks[t] = pak[r];
      }
    }
    const int cntb = cl + (ilast - i0);
#pragma unroll
    for (int r = 0; r <= kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kWaves;
      if (t < cntb)
        biasw[t] = b2 ? __builtin_bit_cast(float, bias2d_key(min(c0 + t, n - 1), a.gh, a.gw, a.cls))
                      : __fadd_rn(pbias[r], 0.0f);
    }
  };

  float theta = -INFINITY;  // admit l > theta
  int cnt = 0;
  // intermediate compactions may leave up to keep + kSlack entries when that
  // still frees room for two more groups
  const bool approx = keep + kSlack <= CAP - 128;
  fetch_chunk(0);
  bool sampled = false;  // theta started from the first chunk's logits
  bool redo = false;     // this row streams again from theta = -inf
  for (int pass = 0; pass < 2; ++pass) {
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    const int cl = min(kChunk, n - c0);
    __syncthreads();
    store_chunk(c0);
    if (c0 + kChunk < n) fetch_chunk(c0 + kChunk);
    __syncthreads();
    if (!live || (pass == 1 && !redo)) continue;
    const int boff = ilast - i;  // bias window index of chunk key t is t + boff
    // Blocks of kG 64-key groups.  The buffer holds at most CAP - 64 entries
    // between groups, so one more group always fits.  Fast path (a full block
    // whose admitted keys keep that bound): kG logits with fixed LDS offsets,
    // then the kG appends.  Otherwise (a partial block, or a block that fills
    // the buffer) the groups go one at a time with bounds checks, compacting
    // when the bound is passed; that path recomputes the logits and runs a few
    // times per query.
    const Code<D>* cp = codes + lane;
    const float* akp = aks + lane;
    const float* bp = biasw + boff + lane;
    const uint32_t* kp = reinterpret_cast<const uint32_t*>(biasw) + lane;  // 2-D: position code of key t
    auto bias_of = [&](const float* w1d, const uint32_t* kpos) {
      return b2 ? bias2d_lookup(tab, qb2, *kpos) : *w1d;
    };
    if (pass == 0 && c0 == 0 && n >= kSampleMinN && cl == kChunk) {
      // Starting threshold from the first chunk's logits (the arithmetic of the loop
      // below): theta keeps about m of them, m the number of kept keys the chunk is
      // expected to hold plus three standard deviations, so the row's keep-th largest
      // logit lies above theta with high probability and the candidate buffer seldom
      // needs compacting.  Only the admissions change: if fewer than `keep` keys pass
      // theta, the row streams again from theta = -inf (below), so the selection stays
      // exact.
      const float e = (float)keep * (float)kChunk / (float)n;
      const int m = (int)ceilf(e + 3.0f * sqrtf(e)) + 2;
      if (2 * m <= kChunk) {
        float sv[kChunk / 64];
#pragma unroll
        for (int r = 0; r < kChunk / 64; ++r)
          sv[r] = canonical_logit(aqv, akp[64 * r], code_dot<D>(cp[64 * r], qq), a.isd, bias_of(bp + 64 * r, kp + 64 * r));
        theta = sample_threshold<kChunk / 64>(sv, m);
        sampled = true;
      }
    }
    for (int s0 = 0; s0 < cl; s0 += 64 * kG) {
      if (s0 + 64 * kG <= cl) {
        float l[kG];
        uint64_t m[kG];
        int tot = 0;
#pragma unroll
        for (int u = 0; u < kG; ++u) {
          l[u] = canonical_logit(aqv, akp[s0 + 64 * u], code_dot<D>(cp[s0 + 64 * u], qq), a.isd,
                                 bias_of(bp + s0 + 64 * u, kp + s0 + 64 * u));
          m[u] = ballot(l[u] > theta);
          tot += __builtin_popcountll(m[u]);
        }
        if (cnt + tot <= CAP - 64) {
#pragma unroll
          for (int u = 0; u < kG; ++u) {
            if (m[u] != 0) {
              if (l[u] > theta)
                buf[cnt + (int)mask_rank(m[u])] =
                    make_uint2(__builtin_bit_cast(uint32_t, l[u]), (uint32_t)(c0 + s0 + 64 * u + lane));
              cnt += __builtin_popcountll(m[u]);
            }
          }
          continue;
        }
      }
      for (int g0 = s0; g0 < min(s0 + 64 * kG, cl); g0 += 64) {
        const int t = g0 + lane;
        const bool ok = t < cl;
        const int tc = ok ? t : 0;
        const float l = canonical_logit(aqv, aks[tc], D - 2 * hamming<D>(codes[tc], qq), a.isd,
                                        bias_of(biasw + tc + boff, reinterpret_cast<const uint32_t*>(biasw) + tc));
        const bool adm = ok && l > theta;
        const uint64_t m = ballot(adm);
        if (m != 0) {
          if (adm) buf[cnt + (int)mask_rank(m)] = make_uint2(__builtin_bit_cast(uint32_t, l), (uint32_t)(c0 + t));
          cnt += __builtin_popcountll(m);
          if (cnt > CAP - 64) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            int kept = approx ? compact_approx<CAP>(buf, cnt, keep, lane, &theta) : -1;
            if (kept < 0) {
              float lm;
              kept = select_compact<CAP>(buf, cand, cnt, keep, lane, &theta, &lm);
            }
            cnt = kept;
          }
        }
      }
    }
  }
  // fewer than `keep` keys above the sampled threshold: stream this row again
  redo = live && pass == 0 && sampled && cnt < keep;
  if (!__syncthreads_or(redo ? 1 : 0)) break;  // uniform over the workgroup
  if (redo) {
    theta = -INFINITY;
    cnt = 0;
  }
  fetch_chunk(0);
  }
  if (!live) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  float lmax;
  float vs;
  cnt = select_compact<CAP>(buf, cand, cnt, keep, lane, &vs, &lmax);  // cnt == keep now
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // ---- softmax over the kept entries (buffer order = ascending key index)
  float z = 0.0f;
  for (int e = lane; e < cnt; e += 64) {
    const float ex = __expf(__builtin_bit_cast(float, buf[e].x) - lmax);
    z += ex;
    buf[e].x = __builtin_bit_cast(uint32_t, ex);
  }
  const float inv_z = 1.0f / wave_sum_f32(z);
  int asum = 0;  // q8: sum of A_q over the kept set
  for (int e = lane; e < a.lcap; e += 64) {
    uint2 ent = e < cnt ? buf[e] : make_uint2(0u, 0u);
    const float p = __builtin_bit_cast(float, ent.x) * inv_z;
    if (VK >= 2) {
      const float qv = fminf(fmaxf(rintf(255.0f * p), 0.0f), 255.0f);
      ent.x = e < cnt ? (uint32_t)qv : 0u;
      asum += (int)ent.x;
    } else {
      ent.x = e < cnt ? __builtin_bit_cast(uint32_t, p) : 0u;
    }
    buf[e] = ent;
    if (a.idx != nullptr && e < cnt) a.idx[row * keep + e] = (int32_t)ent.y;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  if constexpr (VK == 2) {
    // ---- integer A*V with v_dot4_u32_u8: lane (key slot ks = lane / 16, channels c4 .. c4 + 3,
    // c4 = 4 (lane % 16)) takes four kept keys per step, 16 keys per step over the wave.  The
    // four keys' 32-bit reads of their channels are byte-transposed into one word per channel,
    // and V_q + 128 (xor 0x80, unsigned) is multiplied with the packed A_q: the sum is
    // sum A_q V_q + 128 sum A_q, exact in 32 bits (255 * 255 * 1472 < 2^32).
    const int total_a = wave_sum_i32(asum);
    const int c4 = 4 * (lane & 15), ks = lane >> 4;
#pragma unroll
    for (int cb = 0; cb < D / 64; ++cb) {
      const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + (size_t)bh * n * ROWB + cb * 64 + c4;
      uint32_t acc[4] = {0u, 0u, 0u, 0u};
      for (int t = 0; t < a.lcap; t += 16) {
        const uint4 e01 = *reinterpret_cast<const uint4*>(buf + t + 4 * ks);
        const uint4 e23 = *reinterpret_cast<const uint4*>(buf + t + 4 * ks + 2);
        uint32_t w[4];
        w[0] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e01.y * ROWB);
        w[1] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e01.w * ROWB);
        w[2] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e23.y * ROWB);
        w[3] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e23.w * ROWB);
        const uint32_t a4 = e01.x | (e01.z << 8) | (e23.x << 16) | (e23.z << 24);
        const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
        const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
        const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
        const uint32_t vt[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                                __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                                __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                                __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_udot4(a4, vt[c] ^ 0x80808080u, acc[c], false);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] += (uint32_t)__shfl_xor((int)acc[c], 16, 64);
        acc[c] += (uint32_t)__shfl_xor((int)acc[c], 32, 64);
      }
      if (ks == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int ch = cb * 64 + c4 + c;
          const int tot = (int)(acc[c] - 128u * (uint32_t)total_a);
          a.out[row * D + ch] = div255_rn(__fmul_rn((float)tot, a.vscale[(size_t)bh * D + ch]));
        }
      }
    }
    return;
  }

  if constexpr (VK == 3) {
    // ---- 4-bit V: a row is D / 2 bytes of two's-complement nibbles (byte b: channel 2b
    // low, 2b + 1 high).  Lane (key slot ks = lane / 8, channels c8 .. c8 + 7, c8 =
    // 8 (lane % 8)) takes four kept keys per step, 32 keys per step over the wave, with
    // one 32-bit read per key for its eight channels.  Each nibble xor 8 is V_q + 8 in
    // [1, 15]; masked into the bytes of the even and of the odd channels and
    // byte-transposed into one word per channel, it multiplies the packed A_q with
    // v_dot4_u32_u8: sum A_q V_q + 8 sum A_q, exact in 32 bits (255 * 15 * 1472 < 2^32).
    const int total_a = wave_sum_i32(asum);
    const int c8 = 8 * (lane & 7), ks = lane >> 3;
#pragma unroll
    for (int cb = 0; cb < D / 64; ++cb) {
      const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + (size_t)bh * n * ROWB + cb * 32 + c8 / 2;
      uint32_t acc[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      // (the list holds lcap entries, a multiple of 32, zero past the kept ones; two steps
      // per iteration put eight row reads of each lane in flight)
#pragma unroll 2
      for (int t = 0; t < a.lcap; t += 32) {
        const uint4 e01 = *reinterpret_cast<const uint4*>(buf + t + 4 * ks);
        const uint4 e23 = *reinterpret_cast<const uint4*>(buf + t + 4 * ks + 2);
        uint32_t w[4];
        w[0] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e01.y * ROWB) ^ 0x88888888u;
        w[1] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e01.w * ROWB) ^ 0x88888888u;
        w[2] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e23.y * ROWB) ^ 0x88888888u;
        w[3] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)e23.w * ROWB) ^ 0x88888888u;
        const uint32_t a4 = e01.x | (e01.z << 8) | (e23.x << 16) | (e23.z << 24);
        uint32_t ev[4], od[4];  // byte b: channel c8 + 2b (ev) or c8 + 2b + 1 (od) of key k
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          ev[kk] = w[kk] & 0x0f0f0f0fu;
          od[kk] = (w[kk] >> 4) & 0x0f0f0f0fu;
        }
        uint32_t te[4], to[4];  // word m: the four keys' bytes of channel c8 + 2m (te), c8 + 2m + 1 (to)
        transpose_bytes4(ev, te);
        transpose_bytes4(od, to);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[2 * m] = __builtin_amdgcn_udot4(a4, te[m], acc[2 * m], false);
          acc[2 * m + 1] = __builtin_amdgcn_udot4(a4, to[m], acc[2 * m + 1], false);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        acc[c] += (uint32_t)__shfl_xor((int)acc[c], 8, 64);
        acc[c] += (uint32_t)__shfl_xor((int)acc[c], 16, 64);
        acc[c] += (uint32_t)__shfl_xor((int)acc[c], 32, 64);
      }
      if (ks == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int ch = cb * 64 + c8 + c;
          const int tot = (int)(acc[c] - 8u * (uint32_t)total_a);
          a.out[row * D + ch] = div255_rn(__fmul_rn((float)tot, a.vscale[(size_t)bh * D + ch]));
        }
      }
    }
    return;
  }

  // ---- A*V: eight lanes per kept key, eight channels per lane, rows from global memory,
  // per block of 64 channels (head_dim 128 takes two).  U kept keys per lane are
  // fetched before any is used, so U row loads are in flight at once (eight with the
  // larger buffers, whose kept sets are longer and whose two waves per SIMD hide less).
  const int k = lane >> 3, g = lane & 7;
  using Raw = typename std::conditional<VK == 2, uint2, typename std::conditional<VK == 1, uint4, F8>::type>::type;
  using Acc = typename std::conditional<VK == 2, int, float>::type;
  constexpr int U = CAP == kCapBig ? 8 : 4;
#pragma unroll
  for (int cb = 0; cb < D / 64; ++cb) {
    const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + (size_t)bh * n * ROWB + cb * 64 * (ROWB / D);
    auto fetch = [&](uint32_t j) -> Raw {
      return *reinterpret_cast<const Raw*>(vbase + (size_t)j * ROWB + g * sizeof(Raw));
    };
    Acc acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto accum = [&](uint32_t w, const Raw& raw) {
      if constexpr (VK == 2) {
        const int aq8 = (int)w;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[c] += aq8 * (int)(int8_t)(raw.x >> (8 * c));
          acc[4 + c] += aq8 * (int)(int8_t)(raw.y >> (8 * c));
        }
      } else if constexpr (VK == 1) {
        const float p = __builtin_bit_cast(float, w);
        acc[0] = __builtin_fmaf(p, bf16_lo(raw.x), acc[0]);
        acc[1] = __builtin_fmaf(p, bf16_hi(raw.x), acc[1]);
        acc[2] = __builtin_fmaf(p, bf16_lo(raw.y), acc[2]);
        acc[3] = __builtin_fmaf(p, bf16_hi(raw.y), acc[3]);
        acc[4] = __builtin_fmaf(p, bf16_lo(raw.z), acc[4]);
        acc[5] = __builtin_fmaf(p, bf16_hi(raw.z), acc[5]);
        acc[6] = __builtin_fmaf(p, bf16_lo(raw.w), acc[6]);
        acc[7] = __builtin_fmaf(p, bf16_hi(raw.w), acc[7]);
      } else {
        const float p = __builtin_bit_cast(float, w);
        acc[0] = __builtin_fmaf(p, raw.a.x, acc[0]);
        acc[1] = __builtin_fmaf(p, raw.a.y, acc[1]);
        acc[2] = __builtin_fmaf(p, raw.a.z, acc[2]);
        acc[3] = __builtin_fmaf(p, raw.a.w, acc[3]);
        acc[4] = __builtin_fmaf(p, raw.b.x, acc[4]);
        acc[5] = __builtin_fmaf(p, raw.b.y, acc[5]);
        acc[6] = __builtin_fmaf(p, raw.b.z, acc[6]);
        acc[7] = __builtin_fmaf(p, raw.b.w, acc[7]);
      }
    };
    int t = 0;
    for (; t + 8 * U <= a.lcap; t += 8 * U) {
      uint2 ent[U];
      Raw raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) ent[u] = buf[t + 8 * u + k];
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = fetch(ent[u].y);
#pragma unroll
      for (int u = 0; u < U; ++u) accum(ent[u].x, raw[u]);
    }
    for (; t < a.lcap; t += 8) {
      const uint2 ent = buf[t + k];
      accum(ent.x, fetch(ent.y));
    }
    if constexpr (VK == 2) {
      const int tot = reduce_scatter8<int>(acc, k);
      const int ch = cb * 64 + 8 * g + k;
      a.out[row * D + ch] = div255_rn(__fmul_rn((float)tot, a.vscale[(size_t)bh * D + ch]));
    } else {
      a.out[row * D + cb * 64 + 8 * g + k] = reduce_scatter8<float>(acc, k);
    }
  }
}

template <int VK, int D, int W, int CAP, bool B2>
hipError_t launch_b2(StreamKArgs ka, int64_t BH, hipStream_t s) {
  constexpr uint32_t lds = Lds<D, W, CAP>::kTotal;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&topn_stream_kernel<VK, D, W, CAP, B2>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  ka.tiles = (ka.n + W - 1) / W;
  const dim3 grid((unsigned)(BH * ka.tiles));
  hipLaunchKernelGGL((topn_stream_kernel<VK, D, W, CAP, B2>), grid, dim3(64 * W), lds, s, ka);
  return hipGetLastError();
}

template <int VK, int D, int W, int CAP>
hipError_t launch_vk(const StreamKArgs& ka, int64_t BH, hipStream_t s) {
  return ka.brow != nullptr ? launch_b2<VK, D, W, CAP, true>(ka, BH, s) : launch_b2<VK, D, W, CAP, false>(ka, BH, s);
}

// Whether the 768-entry buffers take the kept set and the two-dimensional tables
// (floats; 0 without them).
bool small_cap_fits(int64_t n, int64_t keep, int64_t tab) {
  return keep <= kCapSmall - 64 && tab <= (n > 4096 ? Lds<64, 16>::kTab : Lds<64, 8>::kTab);
}

// 768-entry buffers: sixteen waves per workgroup (one per CU) for the longest
// sequences, where the larger chunks halve the key traffic into LDS; eight (two
// workgroups per CU) below, where the two workgroups' selection and A*V tails overlap.
// Larger kept sets: 1536-entry buffers at eight waves (one workgroup per CU).
template <int VK, int D>
hipError_t launch_w(const StreamKArgs& ka, int64_t tab, int64_t BH, hipStream_t s) {
  if (!small_cap_fits(ka.n, ka.keep, tab)) return launch_vk<VK, D, 8, kCapBig>(ka, BH, s);
  return ka.n > 4096 ? launch_vk<VK, D, 16, kCapSmall>(ka, BH, s) : launch_vk<VK, D, 8, kCapSmall>(ka, BH, s);
}

template <int D>
hipError_t launch_d(const StreamKArgs& ka, int vk, int64_t tab, int64_t BH, hipStream_t s) {
  switch (vk) {
    case 0: return launch_w<0, D>(ka, tab, BH, s);
    case 1: return launch_w<1, D>(ka, tab, BH, s);
    case 2: return launch_w<2, D>(ka, tab, BH, s);
    default: return launch_w<3, D>(ka, tab, BH, s);
  }
}

}  // namespace

bool topn_stream_takes(int64_t n, int64_t keep, int64_t tab) {
  return small_cap_fits(n, keep, tab) || (keep <= kCapBig - 64 && tab <= Lds<64, 8, kCapBig>::kTab);
}

hipError_t launch_topn_stream(const AttnParams& p, hipStream_t s) {
  const int64_t tab = p.brow != nullptr ? bias2d_floats(p.gh, p.gw, p.cls) : 0;
  if ((p.d != 64 && p.d != 128) || !topn_stream_takes(p.n, p.keep, tab)) return hipErrorInvalidValue;
  StreamKArgs ka{};
  ka.qbits = p.qbits;
  ka.kbits = p.kbits;
  ka.aq = p.alpha_q;
  ka.ak = p.alpha_k;
  ka.bias = p.bias;
  ka.brow = p.brow;
  ka.bcol = p.bcol;
  ka.bcls = p.bcls;
  ka.gh = p.gh;
  ka.gw = p.gw;
  ka.cls = p.cls;
  ka.v = p.v;
  ka.vscale = p.vscale;
  ka.out = p.out;
  ka.idx = p.idx;
  ka.H = (int)p.H;
  ka.n = (int)p.n;
  ka.keep = (int)p.keep;
  ka.lcap = (int)((p.keep + 31) / 32 * 32);  // (<= CAP: keep <= CAP - 64)
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  const int64_t BH = p.B * p.H;
  return p.d == 128 ? launch_d<128>(ka, p.v_kind, tab, BH, s) : launch_d<64>(ka, p.v_kind, tab, BH, s);
}

}  // namespace had
