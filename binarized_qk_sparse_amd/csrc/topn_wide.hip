// Top-N binarized attention for long sequences with a large kept set (more keys
// per query than the streaming kernel's on-chip candidate buffer holds, up to
// every key), one wavefront per query.
//
// Same method and arithmetic as the other top-N kernels (Hamming Attention
// Distillation summary: per-query top-N, ties to the lower key index;
// BinaryAttention sections 2.2-2.4: scaled codes, bias, quantized A*V), reached
// threshold first instead of by a candidate buffer:
//  1. the exact N-th largest logit of the row, tau, by radix selection on the
//     order-preserving 32-bit key of the float logit: three passes over the keys,
//     each counting the keys that share the digits found so far into a per-wave
//     histogram of the next 11, 11 and 10 bits;  the count above tau falls out
//     too, and with it `take`, the number of keys equal to tau that are kept
//     (the lowest-indexed ones);
//  2. (quantized A*V) a pass summing exp(l - max) over the kept set, so that
//     A_q = rint(255 p) can be formed with the final normaliser;
//  3. a last pass that keeps l > tau and the first `take` keys with l == tau in
//     ascending key order, appends them to a small per-wave buffer and gathers
//     their V rows into the output whenever it holds 64 of them.
// N >= n keeps every key and skips the selection (one pass for the maximum).
// Keys stream through LDS in chunks shared by the workgroup's waves, which run
// the passes in lockstep.
#include <float.h>

#include <type_traits>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

constexpr int kW = 8;                      // waves (queries) per workgroup
constexpr int kChunk = 128 * kW;           // keys per LDS chunk
constexpr int kPer = kChunk / (64 * kW);   // chunk keys each thread stages
constexpr int kBins = 2048;                // histogram bins per wave (11 bits)
constexpr int kBuf = 128;                  // kept-key buffer entries per wave
constexpr int kTab = 1536;                 // floats of two-dimensional bias tables

struct WideKArgs {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const float* aq;
  const float* ak;
  const float* bias;
  const void* v;
  const float* vscale;
  float* out;
  int32_t* idx;
  int H, n, keep, tiles;
  float isd;
  const float* brow;
  const float* bcol;
  const float* bcls;
  int gh, gw, cls;
};

template <int D>
struct WLds {
  static constexpr uint32_t kCodeOff = 0;                            // Code<D>[kChunk]
  static constexpr uint32_t kAkOff = kCodeOff + kChunk * (D / 8);    // float[kChunk]
  static constexpr uint32_t kBiasOff = kAkOff + kChunk * 4;          // float[kChunk + 64]
  static constexpr uint32_t kHistOff = kBiasOff + (kChunk + 64) * 4;  // uint32[kW][kBins]
  static constexpr uint32_t kBufOff = kHistOff + kW * kBins * 4;     // uint2[kW][kBuf]
  static constexpr uint32_t kTabOff = kBufOff + kW * kBuf * 8;       // float[kTab]
  static constexpr uint32_t kTotal = kTabOff + kTab * 4;
};
static_assert(WLds<128>::kTotal <= 160 * 1024, "LDS");

template <int VK, int D>
constexpr int row_bytes() {
  return VK == 0 ? D * 4 : (VK == 1 ? D * 2 : (VK == 2 ? D : D / 2));
}

// The bin holding the need-th largest entry of a wave's histogram of NB bins
// (higher bin = larger values; 1 <= need <= total) and the number of entries in
// higher bins.  Lane L first sums bins [NB - S (L + 1), NB - S L), starting at a
// lane-dependent offset so that the lanes' reads spread over the banks; an
// exclusive scan over the lanes gives each segment's count from the top; the one
// lane whose segment holds the crossing walks it.
template <int NB>
HAD_DEVICE void hist_select(const uint32_t* hist, int need, int lane, int* bin_out, int* above_out) {
  constexpr int S = NB / 64;
  const int top = NB - S * lane;
  int sum = 0;
#pragma unroll 8
  for (int k = 0; k < S; ++k) sum += (int)hist[top - 1 - ((k + lane) & (S - 1))];
  const int excl = wave_excl_scan_i32(sum);
  const bool here = excl < need && need <= excl + sum;
  const int c = (int)__builtin_ctzll(ballot(here));
  int bin = 0, above = 0;
  if (here) {
    int acc = excl;
    for (int k = 0; k < S; ++k) {
      const int b = top - 1 - k;
      const int h = (int)hist[b];
      if (acc + h >= need) {
        bin = b;
        above = acc;
        break;
      }
      acc += h;
    }
  }
  *bin_out = __builtin_amdgcn_readlane(bin, c);
  *above_out = __builtin_amdgcn_readlane(above, c);
}

// Sum over the eight lanes k = lane / 8 of acc[c] for the lane's channel: lane
// (k, g) ends with the total of entry k (three butterfly halvings).
template <typename T>
HAD_DEVICE T fold8(T (&acc)[8], int k) {
  const bool u4 = k & 4, u2 = k & 2, u1 = k & 1;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const T send = u4 ? acc[c] : acc[c + 4];
    const T stay = u4 ? acc[c + 4] : acc[c];
    acc[c] = stay + __shfl_xor(send, 32, 64);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const T send = u2 ? acc[c] : acc[c + 2];
    const T stay = u2 ? acc[c + 2] : acc[c];
    acc[c] = stay + __shfl_xor(send, 16, 64);
  }
  const T send = u1 ? acc[0] : acc[1];
  const T stay = u1 ? acc[1] : acc[0];
  return stay + __shfl_xor(send, 8, 64);
}

struct F8 {
  float4 a, b;
};

template <int VK, int D, bool B2>
__global__ __launch_bounds__(64 * kW) void topn_wide_kernel(const WideKArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  using L = WLds<D>;
  constexpr int ROWB = row_bytes<VK, D>();
  Code<D>* codes = reinterpret_cast<Code<D>*>(smem + L::kCodeOff);
  float* aks = reinterpret_cast<float*>(smem + L::kAkOff);
  float* biasw = reinterpret_cast<float*>(smem + L::kBiasOff);  // 1-D: bias window; 2-D: key position codes
  float* tab = reinterpret_cast<float*>(smem + L::kTabOff);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L::kHistOff) + wave * kBins;
  uint2* buf = reinterpret_cast<uint2*>(smem + L::kBufOff) + wave * kBuf;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.tiles, tile = wg % a.tiles, hh = bh % a.H;
  const int n = a.n, keep = a.keep;
  const int i0 = tile * kW;
  const int i = i0 + wave;
  const bool live = i < n;  // uniform per wave
  const int ic = live ? i : n - 1;
  const size_t row = (size_t)bh * n + ic;
  const Code<D> qq = load_code<D>(a.qbits, row);
  const float aqv = a.aq != nullptr ? a.aq[row] : 1.0f;
  const int2 qb2 = B2 ? bias2d_query(ic, a.gh, a.gw, a.cls) : make_int2(0, 0);
  if (B2) {
    // the head's tables with each entry + 0 (no -0, as for the 1-D window below);
    // the chunk loop's first barrier orders them before any use
    stage_bias2d(tab, a.brow, a.bcol, a.bcls, hh, a.gh, a.gw, a.cls, (int)threadIdx.x, (int)blockDim.x);
    for (int k = threadIdx.x; k < bias2d_floats(a.gh, a.gw, a.cls); k += blockDim.x) tab[k] = __fadd_rn(tab[k], 0.0f);
  }
  const size_t kb = (size_t)bh * n;
  const float* akg = a.ak != nullptr ? a.ak + (size_t)bh * n : nullptr;
  const int ilast = min(n, i0 + kW) - 1;
  const float* biash = a.bias != nullptr ? a.bias + (size_t)hh * (2 * n - 1) : nullptr;

  // A chunk's key codes, alpha_k and bias window (offsets j - i + n - 1 for the
  // chunk's keys and the workgroup's queries, zero without a table) go global ->
  // registers -> LDS, the next chunk's loads issued before the current one is
  // processed.  + 0 turns a -0 table entry into +0, so no logit is -0 and equal
  // logits have equal order keys.
  Code<D> pcode[kPer];
  float pak[kPer], pbias[kPer + 1];
  auto fetch_chunk = [&](int c0) {
    const int cl = min(kChunk, n - c0);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kW;
      if (t < cl) {
        pcode[r] = load_code<D>(a.kbits, kb + c0 + t);
        pak[r] = akg != nullptr ? akg[c0 + t] : 1.0f;
      }
    }
    const int ob = c0 - ilast + n - 1;
    const int cntb = cl + (ilast - i0);
#pragma unroll
    for (int r = 0; r <= kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kW;
      if (t < cntb) pbias[r] = biash != nullptr ? biash[ob + t] : 0.0f;
    }
  };
  auto store_chunk = [&](int c0) {
    const int cl = min(kChunk, n - c0);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kW;
      if (t < cl) {
        codes[t] = pcode[r];
        aks[t] = pak[r];
      }
    }
    const int cntb = cl + (ilast - i0);
#pragma unroll
    for (int r = 0; r <= kPer; ++r) {
      const int t = (int)threadIdx.x + r * 64 * kW;
      if (t < cntb)
        biasw[t] = B2 ? __builtin_bit_cast(float, bias2d_key(min(c0 + t, n - 1), a.gh, a.gw, a.cls))
                      : __fadd_rn(pbias[r], 0.0f);
    }
  };

  // ---- pass plan: radix levels (or the maximum alone when every key is kept),
  // the normaliser (quantized A*V), the A*V
  const bool all = keep >= n;
  constexpr int kLevel1 = 0, kLevel2 = 1, kLevel3 = 2, kNorm = 3, kAv = 4;
  int plan[5], npass = 0;
  plan[npass++] = kLevel1;
  if (!all) {
    plan[npass++] = kLevel2;
    plan[npass++] = kLevel3;
  }
  if (VK >= 2) plan[npass++] = kNorm;
  plan[npass++] = kAv;

  float lmax = -INFINITY;
  uint32_t prefix = 0, ustar = 0;
  int above = 0, take = 0;
  float inv_z = 0.0f;
  // A*V state: eight lanes per kept key (k = lane / 8), eight channels per lane (g)
  const int k8 = lane >> 3, g8 = lane & 7;
  using Acc = typename std::conditional<VK >= 2, int, float>::type;
  Acc acc[D / 64][8];
#pragma unroll
  for (int cb = 0; cb < D / 64; ++cb)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[cb][c] = 0;
  const uint8_t* vhead = static_cast<const uint8_t*>(a.v) + kb * ROWB;
  // gathers the V rows of buffer entries [0, m) into acc
  auto flush = [&](int m) {
    for (int t = 0; t < m; t += 8) {
      const int e = t + k8;
      if (e < m) {
        const uint2 ent = buf[e];
        const uint8_t* vr = vhead + (size_t)ent.y * ROWB;
#pragma unroll
        for (int cb = 0; cb < D / 64; ++cb) {
          if constexpr (VK == 3) {
            // 4-bit V: eight two's-complement nibbles of one word
            const uint32_t raw = *reinterpret_cast<const uint32_t*>(vr + cb * 32 + 4 * g8);
            const int w = (int)ent.x;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[cb][c] += w * nibble_s4(raw, c);
          } else if constexpr (VK == 2) {
            const uint2 raw = *reinterpret_cast<const uint2*>(vr + cb * 64 + 8 * g8);
            const int w = (int)ent.x;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              acc[cb][c] += w * (int)(int8_t)(raw.x >> (8 * c));
              acc[cb][4 + c] += w * (int)(int8_t)(raw.y >> (8 * c));
            }
          } else if constexpr (VK == 1) {
            const uint4 raw = *reinterpret_cast<const uint4*>(vr + (cb * 64 + 8 * g8) * 2);
            const float w = __builtin_bit_cast(float, ent.x);
            acc[cb][0] = __builtin_fmaf(w, bf16_lo(raw.x), acc[cb][0]);
            acc[cb][1] = __builtin_fmaf(w, bf16_hi(raw.x), acc[cb][1]);
            acc[cb][2] = __builtin_fmaf(w, bf16_lo(raw.y), acc[cb][2]);
            acc[cb][3] = __builtin_fmaf(w, bf16_hi(raw.y), acc[cb][3]);
            acc[cb][4] = __builtin_fmaf(w, bf16_lo(raw.z), acc[cb][4]);
            acc[cb][5] = __builtin_fmaf(w, bf16_hi(raw.z), acc[cb][5]);
            acc[cb][6] = __builtin_fmaf(w, bf16_lo(raw.w), acc[cb][6]);
            acc[cb][7] = __builtin_fmaf(w, bf16_hi(raw.w), acc[cb][7]);
          } else {
            const F8 raw = *reinterpret_cast<const F8*>(vr + (cb * 64 + 8 * g8) * 4);
            const float w = __builtin_bit_cast(float, ent.x);
            acc[cb][0] = __builtin_fmaf(w, raw.a.x, acc[cb][0]);
            acc[cb][1] = __builtin_fmaf(w, raw.a.y, acc[cb][1]);
            acc[cb][2] = __builtin_fmaf(w, raw.a.z, acc[cb][2]);
            acc[cb][3] = __builtin_fmaf(w, raw.a.w, acc[cb][3]);
            acc[cb][4] = __builtin_fmaf(w, raw.b.x, acc[cb][4]);
            acc[cb][5] = __builtin_fmaf(w, raw.b.y, acc[cb][5]);
            acc[cb][6] = __builtin_fmaf(w, raw.b.z, acc[cb][6]);
            acc[cb][7] = __builtin_fmaf(w, raw.b.w, acc[cb][7]);
          }
        }
      }
    }
  };
  int cnt = 0, pos = 0;   // buffer entries; kept keys so far (the index list's position)
  float zsum = 0.0f;      // this lane's share of the normaliser

  for (int p = 0; p < npass; ++p) {
    const int kind = plan[p];
    const bool level = kind <= kLevel3 && !all;
    if (live && level) {
      uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
      for (int k = 0; k < kBins / 256; ++k) h4[k * 64 + lane] = make_uint4(0u, 0u, 0u, 0u);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    int tie_run = 0;  // keys equal to tau met so far (ascending key order)
    zsum = 0.0f;
    fetch_chunk(0);
    for (int c0 = 0; c0 < n; c0 += kChunk) {
      __syncthreads();
      store_chunk(c0);
      if (c0 + kChunk < n) fetch_chunk(c0 + kChunk);
      __syncthreads();
      if (!live) continue;
      const int cl = min(kChunk, n - c0);
      const int boff = ilast - i;  // bias window index of chunk key t is t + boff
      for (int g0 = 0; g0 < cl; g0 += 64) {
        const int t = g0 + lane;
        const bool ok = t < cl;
        const int tc = ok ? t : 0;
        const float b = B2 ? bias2d_lookup(tab, qb2, reinterpret_cast<const uint32_t*>(biasw)[tc]) : biasw[tc + boff];
        const float l = canonical_logit(aqv, aks[tc], code_dot<D>(codes[tc], qq), a.isd, b);
        const uint32_t u = ordered_key(l);
        if (kind == kLevel1) {
          lmax = fmaxf(lmax, ok ? l : -INFINITY);
          if (level && ok) atomicAdd(&hist[u >> 21], 1u);
        } else if (kind == kLevel2) {
          if (ok && (u >> 21) == prefix) atomicAdd(&hist[(u >> 10) & 2047u], 1u);
        } else if (kind == kLevel3) {
          if (ok && (u >> 10) == prefix) atomicAdd(&hist[u & 1023u], 1u);
        } else {
          bool kept = ok;
          if (!all) {
            const bool tie = ok && u == ustar;
            const uint64_t tm = ballot(tie);
            kept = ok && (u > ustar || (tie && tie_run + (int)mask_rank(tm) < take));
            tie_run += __builtin_popcountll(tm);
          }
          const float e = kept ? __expf(l - lmax) : 0.0f;
          if (kind == kNorm) {
            zsum += e;
          } else {
            const uint64_t km = ballot(kept);
            const int slot = (int)mask_rank(km);
            if (kept) {
              uint32_t wbits;
              if constexpr (VK >= 2) {
                wbits = (uint32_t)fminf(fmaxf(rintf(255.0f * (e * inv_z)), 0.0f), 255.0f);
              } else {
                wbits = __builtin_bit_cast(uint32_t, e);
              }
              buf[cnt + slot] = make_uint2(wbits, (uint32_t)(c0 + t));
              if (a.idx != nullptr && pos + slot < keep) a.idx[row * keep + pos + slot] = c0 + t;
            }
            if constexpr (VK < 2) zsum += e;
            const int add = __builtin_popcountll(km);
            cnt += add;
            pos += add;
            if (cnt >= 64) {
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
              flush(64);
              // move the entries past the first 64 to the front
              const uint2 rest = lane + 64 < cnt ? buf[64 + lane] : make_uint2(0u, 0u);
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
              if (lane + 64 < cnt) buf[lane] = rest;
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
              cnt -= 64;
            }
          }
        }
      }
    }
    if (!live) continue;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (kind == kLevel1) {
      lmax = wave_max_f32(lmax);
      if (level) {
        int bin, ab;
        hist_select<kBins>(hist, keep, lane, &bin, &ab);
        prefix = (uint32_t)bin;
        above = ab;
      }
    } else if (kind == kLevel2) {
      int bin, ab;
      hist_select<kBins>(hist, keep - above, lane, &bin, &ab);
      prefix = (prefix << 11) | (uint32_t)bin;
      above += ab;
    } else if (kind == kLevel3) {
      int bin, ab;
      hist_select<1024>(hist, keep - above, lane, &bin, &ab);
      ustar = (prefix << 10) | (uint32_t)bin;
      above += ab;
      take = keep - above;  // keys equal to tau that are kept (>= 1)
    } else if (kind == kNorm) {
      inv_z = 1.0f / wave_sum_f32(zsum);
    }
  }
  if (!live) return;

  // ---- the last buffered keys, then the output
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  flush(cnt);
  float scale = 1.0f;
  if constexpr (VK < 2) scale = 1.0f / wave_sum_f32(zsum);
#pragma unroll
  for (int cb = 0; cb < D / 64; ++cb) {
    const int ch = cb * 64 + 8 * g8 + k8;
    const Acc tot = fold8<Acc>(acc[cb], k8);
    if constexpr (VK >= 2) {
      a.out[row * D + ch] = div255_rn(__fmul_rn((float)tot, a.vscale[(size_t)bh * D + ch]));
    } else {
      a.out[row * D + ch] = tot * scale;
    }
  }
}

template <int VK, int D, bool B2>
hipError_t launch_wide_b2(WideKArgs ka, int64_t BH, hipStream_t s) {
  constexpr uint32_t lds = WLds<D>::kTotal;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&topn_wide_kernel<VK, D, B2>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  if (attr != hipSuccess) return attr;
  ka.tiles = (ka.n + kW - 1) / kW;
  const dim3 grid((unsigned)(BH * ka.tiles));
  hipLaunchKernelGGL((topn_wide_kernel<VK, D, B2>), grid, dim3(64 * kW), lds, s, ka);
  return hipGetLastError();
}

template <int VK, int D>
hipError_t launch_wide_vk(const WideKArgs& ka, int64_t BH, hipStream_t s) {
  return ka.brow != nullptr ? launch_wide_b2<VK, D, true>(ka, BH, s) : launch_wide_b2<VK, D, false>(ka, BH, s);
}

template <int D>
hipError_t launch_wide_d(const WideKArgs& ka, int vk, int64_t BH, hipStream_t s) {
  switch (vk) {
    case 0: return launch_wide_vk<0, D>(ka, BH, s);
    case 1: return launch_wide_vk<1, D>(ka, BH, s);
    case 2: return launch_wide_vk<2, D>(ka, BH, s);
    default: return launch_wide_vk<3, D>(ka, BH, s);
  }
}

}  // namespace

int64_t topn_wide_bias2d_max() { return kTab; }

hipError_t launch_topn_wide(const AttnParams& p, hipStream_t s) {
  if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
  if (p.brow != nullptr && bias2d_floats(p.gh, p.gw, p.cls) > kTab) return hipErrorInvalidValue;
  WideKArgs ka{};
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
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  const int64_t BH = p.B * p.H;
  if (BH * ((p.n + kW - 1) / kW) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  return p.d == 128 ? launch_wide_d<128>(ka, p.v_kind, BH, s) : launch_wide_d<64>(ka, p.v_kind, BH, s);
}

}  // namespace had
