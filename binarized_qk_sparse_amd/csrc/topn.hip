// Top-N binarized attention, one wavefront per query (gfx950, wave64).
//
// Method (Hamming Attention Distillation, summary "main points"/"method"; and
// BinaryAttention sections 2.2-2.4):
//   l_ij = alpha_q alpha_k (d - 2 popcount(q_i XOR k_j)) / sqrt(d) + B_ij
//   S_i  = the N largest l_ij (ties to the lower j)
//   O_i  = sum_{j in S_i} softmax_S(l)_j V_j           (fp32, or uint8 A x int8 V)
//
// Work decomposition.  The work is cut into units of 64 consecutive queries of
// one (batch, head); each workgroup takes a contiguous run of units (logical
// workgroup ids are XCD-remapped so the runs sharing a head sit on one XCD's
// L2).  When its head changes a workgroup stages that head's V rows in LDS --
// bf16 V as fp16 with a per-head power-of-two scale, so the A*V multiply-add
// reads it with v_fma_mix_f32 and needs no conversion instruction -- and each
// wave loads every key's code bits into VGPRs (key j = 64 s + lane lives in
// slot s of lane j % 64).  Per query the wave
//   1. forms the logit of every key (VALU XOR + v_bcnt, two words for d = 64),
//   2. finds the exact top-N threshold without sorting:
//        integer keys (alpha = 1, no bias): the logit is a function of the
//        Hamming distance h in [0, 64], so the threshold is the smallest level
//        tau with #{h <= tau} >= N.  Counts are taken four keys per VALU op on
//        byte-packed distances (SWAR add/and/popcount), starting from the
//        previous query's tau.
//        float keys: bisection on the logit value until at most 64 candidates
//        straddle the threshold, then an exact quickselect among them;
//      ties at the threshold go to the lower key index;
//   3. compacts the kept keys into a per-wave list in LDS (ascending j),
//   4. softmax over the list (fp32), and
//   5. A*V: eight lanes per kept key, eight channels per lane, V read from LDS
//      (16-byte reads), fp32 multiply-add (or int32 on int8 V), then a
//      butterfly reduce-scatter leaves one output channel per lane.
// fp16 staging of bf16 V is exact for every |v| >= 2^(k-17) (k the head's
// scale exponent, 0 unless max|v| >= 2^15) and off by at most 2^(k-25) below,
// so an output moves by at most 2^(k-25) (the probabilities sum to 1).
// The kernel is bound by VALU issue; the only HBM traffic is codes, V and O.
#include <float.h>
#include <limits.h>

#include <algorithm>

#include "had_device.hpp"
#include "had_internal.h"
#include "../../include/had.h"

namespace had {
namespace {

// head_dim D is 64 (codes of two words; every path) or 128 (four words; float keys)
constexpr int kQTile = 64;  // queries per workgroup tile
constexpr int kMaxWaves = 16;
constexpr uint32_t kLdsBytes = 160 * 1024;

struct TopnKArgs {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const float* aq;
  const float* ak;
  const float* bias;
  const void* v;
  const float* vscale;
  float* out;
  int32_t* idx;
  int H, n, keep, lcap, qt, tiles, units, upw;
  // fused entry point: raw Q and K (fp32 or bf16) instead of qbits/kbits/alpha; the
  // head's key codes and scales, the means and the tile's query codes go to LDS at fused_off
  const void* xq;
  const void* xk;
  int qk_bf16, mean;
  uint32_t fused_off;
  float isd;    // float(1/sqrt(d))
  float exp_c;  // 2*isd*log2(e): integer-key exponent per Hamming step
  uint32_t list_off, cand_off, bias_off, red_off, keys_off, trash_off;
  // two-dimensional decomposable bias (brow != NULL; float keys): tables and the
  // key position codes are staged per head at bias_off
  const float* brow;
  const float* bcol;
  const float* bcls;
  int gh, gw, cls;
};

template <int VK, int D>
constexpr int row_bytes() {
  return VK == 0 ? D * 4 : (VK == 1 ? D * 2 : (VK == 2 ? D : D / 2));
}


// Uniform: number of keys j (over all lanes and slots) with hv <= t, t in [0, 64].
// Distances are byte-packed four to a register; a byte b satisfies b > t exactly
// when bit 7 of b + (127 - t) is set (b <= 65, so no byte carries out).
template <int NP>
HAD_DEVICE int count_le(const uint32_t (&P)[NP], int t) {
  const uint32_t add = (uint32_t)(127 - t) * 0x01010101u;
  uint32_t c = 0;
#pragma unroll
  for (int m = 0; m < NP; ++m) c = __builtin_popcount((P[m] + add) & 0x80808080u) + c;
  return NP * 256 - wave_sum_i32((int)c);
}

// Both count_le(t - 1) and count_le(t) with one wave reduction (16-bit halves).
template <int NP>
HAD_DEVICE void count_le2(const uint32_t (&P)[NP], int t, int* c_tm1, int* c_t) {
  const uint32_t add1 = (uint32_t)(128 - t) * 0x01010101u;  // h > t - 1
  const uint32_t add0 = (uint32_t)(127 - t) * 0x01010101u;  // h > t
  uint32_t c1 = 0, c0 = 0;
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    c1 = __builtin_popcount((P[m] + add1) & 0x80808080u) + c1;
    c0 = __builtin_popcount((P[m] + add0) & 0x80808080u) + c0;
  }
  const int both = wave_sum_i32((int)((c0 << 16) + c1));
  *c_tm1 = NP * 256 - (both & 0xffff);
  *c_t = NP * 256 - (both >> 16);
}

template <int NS>
HAD_DEVICE int count_ge_f(const float (&l)[NS], float t) {
  int c = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) c += __builtin_popcountll(ballot(l[s] >= t));
  return c;
}

// Reduce-scatter of the eight key groups' partial sums (group k = lane >> 3
// holds channels 8g..8g+7, g = lane & 7): three butterfly levels over lane bits
// 5, 4, 3 leave lane (k, g) with the total of channel 8g + k.
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
  T other;
  if constexpr (sizeof(T) == 4 && T(0.5) != T(0)) {
    other = dpp_f<kRowRor8>(snd);  // lane ^ 8 within the 16-lane row
  } else {
    other = dpp_i<kRowRor8>(snd);
  }
  return kp + other;
}

// Streams `total` bytes (a multiple of 16) of global memory through f(offset,
// 16 bytes), eight 16-byte loads in flight per thread before any is used.
template <typename F>
HAD_DEVICE void for_each16(const uint8_t* __restrict__ src, uint32_t total, F f) {
  const uint32_t step = blockDim.x * 16u;
  for (uint32_t base = threadIdx.x * 16u; base < total; base += 8u * step) {
    uint4 w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t o = base + k * step;
      w[k] = o < total ? *reinterpret_cast<const uint4*>(src + o) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t o = base + k * step;
      if (o < total) f(o, w[k]);
    }
  }
}

// One 32-channel word of a token's code and the float64 sum of |y| over those
// channels, y = x (plain sign) or fl(x - mu) (mean-centred), summed in channel
// order: the arithmetic of had_pack, so both give the same bits.
HAD_DEVICE uint32_t code_word(const void* x, bool bf16, size_t row, int D, int part, const float* mu, double* asum) {
  double s = 0.0;
  uint32_t w = 0;
#pragma unroll 2
  for (int k = 0; k < 4; ++k) {
    float v[8];
    const size_t e = row * D + 32 * part + 8 * k;
    if (bf16) {
      const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e);
      v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
      v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    } else {
      const float4 q0 = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + e);
      const float4 q1 = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + e + 4);
      v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
      v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
    }
    if (mu != nullptr) {
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = __fsub_rn(v[c], mu[32 * part + 8 * k + c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) s += fabs((double)v[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) w |= (uint32_t)(v[c] < 0.0f) << (8 * k + c);
  }
  *asum = s;
  return w;
}

// EXT: 0 plain; 1 (float keys only) the two-dimensional bias, a separate instance so
// that the 1-D path carries none of its code; 2 the fused entry point (raw Q and K
// binarized on chip, fp32 or bf16 V)
template <int NS, bool FK, int VK, bool PAD, int D, int EXT = 0>
__global__ __launch_bounds__(1024) void topn_resident_kernel(const TopnKArgs a) {
  static_assert(D == 64 || (D == 128 && FK), "head_dim 128 takes the float-key path");
  constexpr bool B2 = EXT == 1;
  constexpr bool fused = EXT == 2;
  constexpr int W = D / 32;
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int ROWB = row_bytes<VK, D>();
  constexpr int NP = (NS + 3) / 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int n = a.n, keep = a.keep;
  const int u0 = (int)xcd_remap(blockIdx.x, gridDim.x) * a.upw;
  const int u1 = min(a.units, u0 + a.upw);
  uint2* list = reinterpret_cast<uint2*>(smem + a.list_off) + wave * a.lcap;
  uint2* cand = reinterpret_cast<uint2*>(smem + a.cand_off) + wave * 64;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem + a.keys_off) + wave * a.lcap;
  uint32_t* trash = reinterpret_cast<uint32_t*>(smem + a.trash_off) + wave * 64;
  float* biasw = reinterpret_cast<float*>(smem + a.bias_off);
  uint32_t* red = reinterpret_cast<uint32_t*>(smem + a.red_off);
  // fused: the head's key code words [n][W] and key scales [n], the means of Q and K
  // [2][D], and the unit's query code words [64][W] and query scales [64]
  uint32_t* fcode = reinterpret_cast<uint32_t*>(smem + a.fused_off);
  float* falpha = reinterpret_cast<float*>(fcode + (size_t)n * W);
  float* fmu = falpha + n;
  uint32_t* fqcode = reinterpret_cast<uint32_t*>(fmu + 2 * D);
  float* fqalpha = reinterpret_cast<float*>(fqcode + 64 * W);
  uint32_t kw[W][NS];  // key code words: word w of slot s
  float akv[NS];
  int staged = -1;
  float vmul = 1.0f;  // undoes the fp16 staging scale of V
  int tau_prev = 27;  // Hamming-level guess; each query starts from the last one's
  float wlo = 0.0f, whi = 0.0f;  // float keys: the last query's final threshold bracket (empty: none)
  Code<D> qnext{};
  float aqnext = 1.0f;
  {
    const int nbh = u0 / a.tiles, ni0 = (u0 % a.tiles) * a.qt;
    const bool ok = u0 < u1 && ni0 + lane < n;
    const size_t nrow = (size_t)nbh * n + ni0 + lane;
    if (!fused) {
      qnext = load_code<D>(a.qbits, ok ? nrow : 0);
      aqnext = (FK && a.aq != nullptr && ok) ? a.aq[nrow] : 1.0f;
    }
  }

  for (int u = u0; u < u1; ++u) {
    const int bh = u / a.tiles, tile = u % a.tiles, hh = bh % a.H;
    const int i0 = tile * a.qt, i1 = min(n, i0 + a.qt);
    const bool restage = bh != staged;                       // uniform over the workgroup
    const bool sync = restage || fused || (FK && a.bias != nullptr);  // LDS contents change this unit
    constexpr bool b2 = FK && B2;
    if (sync) __syncthreads();  // every wave is done with the previous unit's LDS data
    if (restage) {
      staged = bh;
      if constexpr (fused) {
        // ---- binarize this head's queries and keys (mean-centred: after the means of Q
        // and K) with had_pack's arithmetic and summation order
        const bool qb = a.qk_bf16 != 0;
        const int t = (int)threadIdx.x;
        if (a.mean) {
          // column sums in float64: thread tt < 256 of set x takes channels 8 cg .. 8 cg + 7
          // of rows r + RPP k (n <= 256: one chunk); the V area holds the RPP x D partials
          // of each set; with 512 threads or more Q and K are summed together
          constexpr int RPP = 256 / (D / 8);
          const int nset = min(2, (int)blockDim.x / 256);
          for (int x0 = 0; x0 < 2; x0 += nset) {
            const int x = x0 + t / 256, tt = t % 256, r = tt / (D / 8), cg = tt % (D / 8);
            double* part = reinterpret_cast<double*>(smem) + (x - x0) * RPP * D;
            if (x < x0 + nset) {
              const void* src = x == 0 ? a.xq : a.xk;
              double cs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
              for (int k = 0; k < 256 / RPP; ++k) {
                const int row = r + RPP * k;
                if (row < n) {
                  float v[8];
                  const size_t e = ((size_t)bh * n + row) * D + 8 * cg;
                  if (qb) {
                    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + e);
                    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
                    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
                  } else {
                    const float* pf = static_cast<const float*>(src) + e;
                    const float4 w0 = *reinterpret_cast<const float4*>(pf);
                    const float4 w1 = *reinterpret_cast<const float4*>(pf + 4);
                    v[0] = w0.x; v[1] = w0.y; v[2] = w0.z; v[3] = w0.w;
                    v[4] = w1.x; v[5] = w1.y; v[6] = w1.z; v[7] = w1.w;
                  }
#pragma unroll
                  for (int c = 0; c < 8; ++c) cs[c] += (double)v[c];
                }
              }
#pragma unroll
              for (int c = 0; c < 8; ++c) part[r * D + 8 * cg + c] = cs[c];
            }
            __syncthreads();
            if (t < nset * D) {
              const int xx = x0 + t / D, c = t % D;
              const double* pp = reinterpret_cast<const double*>(smem) + (xx - x0) * RPP * D;
              double acc = 0.0;
              for (int rp = 0; rp < RPP; ++rp) acc += pp[rp * D + c];
              fmu[xx * D + c] = (float)((0.0 + acc) / (double)n);
            }
            __syncthreads();
          }
        }
        // key codes, then this unit's query codes, in one pass: W consecutive lanes per
        // row (one word each), as had_pack's rows kernel; dead lanes read a valid row
        const int nk = n * W, nall = nk + a.qt * W;
        for (int it0 = 0; it0 < nall; it0 += (int)blockDim.x) {
          const int it = it0 + t;
          const bool key = it < nk;
          const int j = key ? it / W : min(i0 + (min(it, nall - 1) - nk) / W, n - 1);
          double sm;
          const uint32_t w = code_word(key ? a.xk : a.xq, qb, (size_t)bh * n + j, D, t % W,
                                       a.mean ? fmu + (key ? D : 0) : nullptr, &sm);
#pragma unroll
          for (int off = 1; off < W; off <<= 1) sm += __shfl_xor(sm, off, 64);
          const float al = a.mean ? (float)(sm / (double)D) : 1.0f;
          if (key) {
            fcode[it] = w;
            if (t % W == 0) falpha[j] = al;
          } else if (it < nall) {
            fqcode[it - nk] = w;
            if (t % W == 0) fqalpha[(it - nk) / W] = al;
          }
        }
        __syncthreads();  // (the V area's partials are dead; the codes are in place)
      }
      // ---- this head's V rows into LDS (16 bytes per thread and step)
      const uint8_t* src = static_cast<const uint8_t*>(a.v) + (size_t)bh * n * ROWB;
      const uint32_t total = (uint32_t)n * ROWB;
      if (VK == 1) {
        // bf16 -> fp16 with a power-of-two scale 2^-k chosen so max|v| 2^-k < 2^15
        uint32_t mx = 0;
        for_each16(src, total, [&](uint32_t, const uint4& w) {
          mx = max(mx, max(max(w.x & 0x7fffu, w.x >> 16 & 0x7fffu), max(w.y & 0x7fffu, w.y >> 16 & 0x7fffu)));
          mx = max(mx, max(max(w.z & 0x7fffu, w.z >> 16 & 0x7fffu), max(w.w & 0x7fffu, w.w >> 16 & 0x7fffu)));
        });
        mx = wave_max_u32(mx);
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        mx = 0;
        for (int w = 0; w < nwaves; ++w) mx = max(mx, red[w]);
        const float vmax = __builtin_bit_cast(float, mx << 16);
        int e;
        (void)frexpf(vmax, &e);  // vmax < 2^e
        const int kexp = max(0, e - 15);
        const float down = ldexpf(1.0f, -kexp);
        vmul = ldexpf(1.0f, kexp);
        for_each16(src, total, [&](uint32_t o, const uint4& w) {
          uint4 h;
          h.x = pack_half2(bf16_lo(w.x) * down, bf16_hi(w.x) * down);
          h.y = pack_half2(bf16_lo(w.y) * down, bf16_hi(w.y) * down);
          h.z = pack_half2(bf16_lo(w.z) * down, bf16_hi(w.z) * down);
          h.w = pack_half2(bf16_lo(w.w) * down, bf16_hi(w.w) * down);
          *reinterpret_cast<uint4*>(smem + o) = h;
        });
      } else {
        for_each16(src, total, [&](uint32_t o, const uint4& w) { *reinterpret_cast<uint4*>(smem + o) = w; });
      }
      // ---- key codes.  Float keys: slot s of this lane is key 64 s + lane.  Integer
      // keys: slot s of lane l is key NS l + s (a lane holds consecutive keys).
      // PAD: keys j >= n are padding.
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = FK ? 64 * s + lane : NS * lane + s;
        const bool ok = !PAD || j < n;
        Code<D> kk;
        if constexpr (fused) {
#pragma unroll
          for (int w = 0; w < W; ++w) kk.w[w] = fcode[(size_t)(ok ? j : 0) * W + w];
        } else {
          kk = load_code<D>(a.kbits, (size_t)bh * n + (ok ? j : 0));
        }
#pragma unroll
        for (int w = 0; w < W; ++w) kw[w][s] = ok ? kk.w[w] : 0u;
        if (fused)
          akv[s] = (FK && ok) ? falpha[j] : 1.0f;
        else
          akv[s] = (FK && ok && a.ak != nullptr) ? a.ak[(size_t)bh * n + j] : 1.0f;
      }
    }
    // ---- two-dimensional bias: this head's tables, then the key position codes
    if (b2 && restage) {
      stage_bias2d(biasw, a.brow, a.bcol, a.bcls, hh, a.gh, a.gw, a.cls, (int)threadIdx.x, (int)blockDim.x);
      uint32_t* kp = reinterpret_cast<uint32_t*>(biasw + bias2d_floats(a.gh, a.gw, a.cls));
      for (int j = threadIdx.x; j < n; j += blockDim.x) kp[j] = bias2d_key(j, a.gh, a.gw, a.cls);
    }
    // ---- the bias offsets this tile touches: o = j - i + n - 1 in [n - i1, 2n - 2 - i0]
    const int ob = n - i1;
    if (FK && a.bias != nullptr) {
      const int cnt = n + (i1 - i0) - 1;
      const float* src = a.bias + (size_t)hh * (2 * n - 1) + ob;
      for (int o = threadIdx.x; o < cnt; o += 2 * blockDim.x) {
        const int o2 = o + blockDim.x;
        const float b0 = src[o];
        const float b1 = o2 < cnt ? src[o2] : 0.0f;
        biasw[o] = b0;
        if (o2 < cnt) biasw[o2] = b1;
      }
    }
    // ---- the tile's query codes (and scales), one query per lane, read back with
    // v_readlane; the next unit's are fetched now so their latency hides behind this unit
    if (fused && !restage) {
      // this unit's query codes and scales (with the head's means): the first waves take
      // W lanes per query row as for the keys
      const int t = (int)threadIdx.x;
      if (t < (a.qt * W + 63) / 64 * 64) {  // whole waves (the sums cross lanes)
        const int r = t / W, i = min(i0 + r, n - 1);
        double sm;
        const uint32_t w = code_word(a.xq, a.qk_bf16 != 0, (size_t)bh * n + i, D, t % W, a.mean ? fmu : nullptr, &sm);
#pragma unroll
        for (int off = 1; off < W; off <<= 1) sm += __shfl_xor(sm, off, 64);
        fqcode[t] = w;
        if (t % W == 0) fqalpha[r] = a.mean ? (float)(sm / (double)D) : 1.0f;
      }
    }
    Code<D> qlane = qnext;
    float aqlane = aqnext;
    if (!fused && u + 1 < u1) {
      const int nbh = (u + 1) / a.tiles, ni0 = ((u + 1) % a.tiles) * a.qt;
      const bool ok = ni0 + lane < n;
      const size_t nrow = (size_t)nbh * n + ni0 + lane;
      qnext = load_code<D>(a.qbits, ok ? nrow : 0);
      aqnext = (FK && a.aq != nullptr && ok) ? a.aq[nrow] : 1.0f;
    }
    if (sync) __syncthreads();
    if constexpr (fused) {
#pragma unroll
      for (int w = 0; w < W; ++w) qlane.w[w] = fqcode[lane * W + w];
      aqlane = fqalpha[lane];
    }

  for (int i = i0 + wave; i < i1; i += nwaves) {
    const size_t row = (size_t)bh * n + i;
    uint32_t qw[W];
#pragma unroll
    for (int w = 0; w < W; ++w) qw[w] = __builtin_amdgcn_readlane(qlane.w[w], i - i0);
    float ref = 0.0f;  // float keys: softmax reference (the row's largest logit)
    int tref = 0;      // integer keys: softmax reference level (the threshold tau)

    if (!FK) {
      // ------------------------------------------------ integer keys
      uint32_t hv[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        hv[s] = __builtin_popcount(kw[1][s] ^ qw[1]) + __builtin_popcount(kw[0][s] ^ qw[0]);
        if (PAD && NS * lane + s >= n) hv[s] = 65u;  // above every real distance
      }
      uint32_t P[NP];
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        uint32_t b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = (4 * m + q < NS) ? hv[4 * m + q] : 65u;
        P[m] = ((b[3] << 8 | b[2]) << 16) | (b[1] << 8 | b[0]);
      }
      int tau, less;
      if (keep >= n) {
        tau = 65;  // every real key is below the padding level
        less = keep;
      } else {
        // invariant once bracketed: count_le(lo) = clo < keep <= count_le(hi)
        int lo, hi, clo;
        const int t = tau_prev;  // in [1, 64]
        int ctm1, ct;
        count_le2<NP>(P, t, &ctm1, &ct);
        if (ctm1 < keep && ct >= keep) {
          lo = t - 1;
          hi = t;
          clo = ctm1;
        } else if (ct < keep) {
          lo = t;
          clo = ct;
          hi = 64;
        } else {
          hi = t - 1;
          lo = -1;
          clo = 0;
        }
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          const int cm = count_le<NP>(P, mid);
          if (cm >= keep) {
            hi = mid;
          } else {
            lo = mid;
            clo = cm;
          }
        }
        tau = hi;
        less = clo;
        tau_prev = max(tau, 1);
      }
      // ---- tie cutoff and compaction, all in VALU (no per-slot scalar work).
      // Keys are lane-major, so ascending j is lane order, then slot order.  Per lane:
      // c_lt keys below tau and c_eq keys at tau (SWAR counts on the packed
      // distances); a prefix over lanes of c_eq hands each lane `take` of the
      // keep - less keys at tau (lowest j first); a prefix of c_lt + take gives the
      // lane's first list position.
      const int r = keep - less;
      const uint32_t ad0 = (uint32_t)(128 - tau) * 0x01010101u;  // bit 7: h >= tau
      const uint32_t ad1 = (uint32_t)(127 - tau) * 0x01010101u;  // bit 7: h >= tau + 1
      int c_lt = 0, c_eq = 0;
      uint32_t eqw[NP];
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const uint32_t ge0 = (P[m] + ad0) & 0x80808080u;
        const uint32_t ge1 = (P[m] + ad1) & 0x80808080u;
        eqw[m] = ge0 ^ ge1;
        c_lt += 4 - __builtin_popcount(ge0);
        c_eq += __builtin_popcount(eqw[m]);
      }
      const int eq_before = wave_excl_scan_i32(c_eq);
      const int take = min(max(r - eq_before, 0), c_eq);
      const int lbase = wave_excl_scan_i32(c_lt + take);
      // slot of this lane's take-th key at tau: the number of slots whose running
      // count of keys at tau is still below take (byte-wise prefix counts)
      int scut = 0;
      uint32_t carry = 0;
      const uint32_t adt = (uint32_t)(128 - take) * 0x01010101u;  // bit 7: count >= take
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        uint32_t x = eqw[m] >> 7;  // 0/1 per byte
        x += x << 8;
        x += x << 16;
        x += carry * 0x01010101u;
        carry = x >> 24;
        scut += 4 - __builtin_popcount((x + adt) & 0x80808080u);
      }
      // selected: (h, s) <= (tau, scut) lexicographically, or h < tau when take == 0
      // (a strict bound, so tau = 0 with take = 0 selects nothing)
      const uint32_t lim = take > 0 ? (((uint32_t)tau << 5) | (uint32_t)scut) + 1u : ((uint32_t)tau << 5);
      int pos = lbase;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint32_t w = (hv[s] << 5) | (uint32_t)s;
        const bool sel = w < lim;
        uint32_t* dst = sel ? keys + pos : trash + lane;
        *dst = (w << 6) | (uint32_t)lane;  // h, slot, lane: j = NS * lane + slot
        pos += sel ? 1 : 0;
      }
      tref = tau;
    } else {
      // ------------------------------------------------ float keys
      const float aqv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, aqlane), i - i0));
      float lg[NS];
      const int boff = n - 1 - ob - i;  // bias window index of key j is j + boff
      const int2 qb2 = b2 ? bias2d_query(i, a.gh, a.gw, a.cls) : make_int2(0, 0);
      const uint32_t* kposs = reinterpret_cast<const uint32_t*>(biasw + (b2 ? bias2d_floats(a.gh, a.gw, a.cls) : 0));
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = 64 * s + lane;
        int hd = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) hd = __builtin_popcount(kw[w][s] ^ qw[w]) + hd;
        const bool ok = !PAD || j < n;
        const float bias = !ok ? 0.0f
                               : (b2 ? bias2d_lookup(biasw, qb2, kposs[j])
                                     : (a.bias != nullptr ? biasw[j + boff] : 0.0f));
        const float l = canonical_logit(aqv, akv[s], D - 2 * hd, a.isd, bias);
        lg[s] = ok ? __fadd_rn(l, 0.0f) : -INFINITY;  // -0 and +0 compare equal
      }
      float vstar;
      int jstar;
      float lmax = -INFINITY;
#pragma unroll
      for (int s = 0; s < NS; ++s) lmax = fmaxf(lmax, lg[s]);
      lmax = wave_max_f32(lmax);
      ref = lmax;
      if (keep >= n) {
        vstar = -INFINITY;  // everything real is kept
        jstar = INT_MAX;
      } else {
        auto row_min = [&]() {
          float m = INFINITY;
#pragma unroll
          for (int s = 0; s < NS; ++s) m = fminf(m, lg[s] == -INFINITY ? INFINITY : lg[s]);
          return -wave_max_f32(-m);
        };
        int need;  // keys still to take at value vstar (lowest j first)
        const int ctop = count_ge_f<NS>(lg, lmax);
        if (ctop >= keep) {
          vstar = lmax;
          need = keep;
        } else {
          // invariant: cnt(>= lo) >= keep > cnt(>= hi).  The search starts from the last
          // query's final bracket when its counts keep the invariant on this row (neighbouring
          // queries have close thresholds), else from [min, max] of the row.
          float lo, hi;
          int clo, chi;
          if (wlo < whi && wlo < lmax) {
            const float b = fminf(whi, lmax);
            const int ca = count_ge_f<NS>(lg, wlo);
            if (ca >= keep) {
              const int cb = b == lmax ? ctop : count_ge_f<NS>(lg, b);
              if (cb < keep) {
                lo = wlo, clo = ca, hi = b, chi = cb;
              } else {
                lo = b, clo = cb, hi = lmax, chi = ctop;
              }
            } else {
              lo = row_min(), clo = n, hi = wlo, chi = ca;
            }
          } else {
            lo = row_min(), clo = n, hi = lmax, chi = ctop;
          }
          bool split = true;
          while (clo - chi > 64) {
            const float mid = 0.5f * lo + 0.5f * hi;
            if (!(mid > lo && mid < hi)) {
              split = false;
              break;
            }
            const int cm = count_ge_f<NS>(lg, mid);
            if (cm >= keep) {
              lo = mid;
              clo = cm;
            } else {
              hi = mid;
              chi = cm;
            }
          }
          wlo = lo;
          whi = hi;
          if (!split) {
            vstar = lo;  // hi is the next float after lo: every candidate equals lo
            need = keep - chi;
          } else {
            // compact the candidates lo <= l < hi (at most 64) into one per lane
            int cb = 0;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              const bool c = lg[s] >= lo && lg[s] < hi;
              const uint64_t m = ballot(c);
              const int pos = cb + (int)mask_rank(m);
              if (c && pos < 64) cand[pos] = make_uint2(ordered_key(lg[s]), (uint32_t)(64 * s + lane));
              cb += __builtin_popcountll(m);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const uint32_t ck = lane < cb ? cand[lane].x : 0u;
            const int rr = keep - chi;  // how many candidates to take
            // the rr-th largest candidate (lanes >= cb hold 0, below every key)
            const uint32_t L = wave_select_desc(ck, cb, rr);
            vstar = from_ordered_key(L);
            need = keep - chi - __builtin_popcountll(ballot(ck > L));
          }
        }
        // the need-th key (ascending j) with l == vstar
        jstar = INT_MAX;
        int seen = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint64_t Em = ballot(lg[s] == vstar);
          const int e = __builtin_popcountll(Em);
          if (jstar == INT_MAX && seen + e >= need) {
            uint64_t x = Em;
            for (int k = 0; k < need - seen - 1; ++k) x &= x - 1;
            jstar = 64 * s + (int)__builtin_ctzll(x);
          }
          seen += e;
        }
      }
      // ---- compaction of l > vstar, or l == vstar with j <= jstar
      int base = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = 64 * s + lane;
        const bool sel = (!PAD || j < n) && (lg[s] > vstar || (lg[s] == vstar && j <= jstar));
        const uint64_t Sm = ballot(sel);
        if (sel) {
          const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(Sm >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)Sm, (uint32_t)base));
          if (pos < a.lcap) list[pos] = make_uint2((uint32_t)j, __builtin_bit_cast(uint32_t, lg[s]));
        }
        base += __builtin_popcountll(Sm);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    // ---------------------------------------------------- softmax over the kept list
    // float keys: e_j = exp(l_j - max l).  Integer keys: e_j = exp(l_j - l(tau)) =
    // exp(2 (tau - h_j) / sqrt(d)); the shift cancels in the normalisation and
    // stays below exp(2 (d + 1) / sqrt(d)), far from float overflow.
    // Unnormalised weights go to the list; fp32 paths scale the output by 1/Z at
    // the end, the int8 path needs p itself for A_q and normalises here.
    float z = 0.0f;
    for (int e = lane; e < a.lcap; e += 64) {
      uint2 ent = make_uint2(0u, 0u);
      if (e < keep) {
        float ex;
        if (FK) {
          ent = list[e];
          ex = __expf(__builtin_bit_cast(float, ent.y) - ref);
        } else {
          const uint32_t key = keys[e];  // h << 11 | slot << 6 | lane
          ent.x = (uint32_t)NS * (key & 63u) + ((key >> 6) & 31u);
          ex = exp2f((float)(tref - (int)(key >> 11)) * a.exp_c);
        }
        z += ex;
        ent.y = __builtin_bit_cast(uint32_t, ex);
        if (a.idx != nullptr) a.idx[row * keep + e] = (int32_t)ent.x;
      }
      list[e] = ent;
    }
    const float inv_z = __builtin_amdgcn_rcpf(wave_sum_f32(z));
    if (VK >= 2) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      for (int e = lane; e < keep; e += 64) {
        const float p = __builtin_bit_cast(float, list[e].y) * inv_z;
        list[e].y = (uint32_t)fminf(fmaxf(rintf(255.0f * p), 0.0f), 255.0f);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    // ---------------------------------------------------- A*V
    // (per block of 64 channels: head_dim 128 takes two)
    const int k = lane >> 3, g = lane & 7;
#pragma unroll
    for (int cb = 0; cb < D / 64; ++cb) {
      const uint8_t* const vrow0 = smem + cb * 64 * ROWB / D;
      if (VK == 3) {
        // 4-bit V: the lane's eight channels are eight two's-complement nibbles of one word
        int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int t = 0; t < a.lcap; t += 32) {
          uint2 ent[4];
          uint32_t raw[4];
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) ent[u4] = list[t + 8 * u4 + k];
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) raw[u4] = *reinterpret_cast<const uint32_t*>(vrow0 + ent[u4].x * ROWB + g * 4);
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) {
            const int aq8 = (int)ent[u4].y;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] += aq8 * nibble_s4(raw[u4], c);
          }
        }
        const int tot = reduce_scatter8<int>(acc, k);
        const int ch = cb * 64 + 8 * g + k;
        const float sc = a.vscale[(size_t)bh * D + ch];
        a.out[row * D + ch] = div255_rn(__fmul_rn((float)tot, sc));
      } else if (VK == 2) {
        int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int t = 0; t < a.lcap; t += 32) {
          uint2 ent[4], raw[4];
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) ent[u4] = list[t + 8 * u4 + k];
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) raw[u4] = *reinterpret_cast<const uint2*>(vrow0 + ent[u4].x * ROWB + g * 8);
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) {
            const int aq8 = (int)ent[u4].y;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              acc[c] += aq8 * (int)(int8_t)(raw[u4].x >> (8 * c));
              acc[4 + c] += aq8 * (int)(int8_t)(raw[u4].y >> (8 * c));
            }
          }
        }
        const int tot = reduce_scatter8<int>(acc, k);
        const int ch = cb * 64 + 8 * g + k;
        const float sc = a.vscale[(size_t)bh * D + ch];
        a.out[row * D + ch] = div255_rn(__fmul_rn((float)tot, sc));
      } else {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        // four entries per group in flight: their list reads, then their row reads, then the math
        for (int t = 0; t < a.lcap; t += 32) {
          uint2 ent[4];
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) ent[u4] = list[t + 8 * u4 + k];
          if (VK == 1) {  // fp16 rows: the widening folds into v_fma_mix_f32
            uint4 raw[4];
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) raw[u4] = *reinterpret_cast<const uint4*>(vrow0 + ent[u4].x * ROWB + g * 16);
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
              const float p = __builtin_bit_cast(float, ent[u4].y);
              const half2v h0 = __builtin_bit_cast(half2v, raw[u4].x), h1 = __builtin_bit_cast(half2v, raw[u4].y);
              const half2v h2 = __builtin_bit_cast(half2v, raw[u4].z), h3 = __builtin_bit_cast(half2v, raw[u4].w);
              acc[0] = __builtin_fmaf(p, (float)h0.x, acc[0]);
              acc[1] = __builtin_fmaf(p, (float)h0.y, acc[1]);
              acc[2] = __builtin_fmaf(p, (float)h1.x, acc[2]);
              acc[3] = __builtin_fmaf(p, (float)h1.y, acc[3]);
              acc[4] = __builtin_fmaf(p, (float)h2.x, acc[4]);
              acc[5] = __builtin_fmaf(p, (float)h2.y, acc[5]);
              acc[6] = __builtin_fmaf(p, (float)h3.x, acc[6]);
              acc[7] = __builtin_fmaf(p, (float)h3.y, acc[7]);
            }
          } else {
            float4 r0[4], r1[4];
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
              r0[u4] = *reinterpret_cast<const float4*>(vrow0 + ent[u4].x * ROWB + g * 32);
              r1[u4] = *reinterpret_cast<const float4*>(vrow0 + ent[u4].x * ROWB + g * 32 + 16);
            }
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
              const float p = __builtin_bit_cast(float, ent[u4].y);
              acc[0] = __builtin_fmaf(p, r0[u4].x, acc[0]);
              acc[1] = __builtin_fmaf(p, r0[u4].y, acc[1]);
              acc[2] = __builtin_fmaf(p, r0[u4].z, acc[2]);
              acc[3] = __builtin_fmaf(p, r0[u4].w, acc[3]);
              acc[4] = __builtin_fmaf(p, r1[u4].x, acc[4]);
              acc[5] = __builtin_fmaf(p, r1[u4].y, acc[5]);
              acc[6] = __builtin_fmaf(p, r1[u4].z, acc[6]);
              acc[7] = __builtin_fmaf(p, r1[u4].w, acc[7]);
            }
          }
        }
        a.out[row * D + cb * 64 + 8 * g + k] = reduce_scatter8<float>(acc, k) * (vmul * inv_z);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  }
}

template <int NS, bool FK, int VK, bool PAD, int D, int EXT>
hipError_t launch_inst(const TopnKArgs& ka, dim3 grid, dim3 block, uint32_t lds, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&topn_resident_kernel<NS, FK, VK, PAD, D, EXT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((topn_resident_kernel<NS, FK, VK, PAD, D, EXT>), grid, block, lds, s, ka);
  return hipGetLastError();
}

template <int NS, bool FK, int VK, bool PAD, int D>
hipError_t launch_one(const TopnKArgs& ka, dim3 grid, dim3 block, uint32_t lds, hipStream_t s) {
  if constexpr (FK) {
    if (ka.brow != nullptr) return launch_inst<NS, FK, VK, PAD, D, 1>(ka, grid, block, lds, s);
  }
  if constexpr (VK < 2) {
    if (ka.xk != nullptr) return launch_inst<NS, FK, VK, PAD, D, 2>(ka, grid, block, lds, s);
  }
  return launch_inst<NS, FK, VK, PAD, D, 0>(ka, grid, block, lds, s);
}

template <int NS, bool FK, int VK, int D>
hipError_t launch_pad(const TopnKArgs& ka, bool pad, dim3 grid, dim3 block, uint32_t lds, hipStream_t s) {
  return pad ? launch_one<NS, FK, VK, true, D>(ka, grid, block, lds, s)
             : launch_one<NS, FK, VK, false, D>(ka, grid, block, lds, s);
}

template <int NS, bool FK, int D>
hipError_t launch_vk(const TopnKArgs& ka, int vk, bool pad, dim3 grid, dim3 block, uint32_t lds, hipStream_t s) {
  switch (vk) {
    case 0: return launch_pad<NS, FK, 0, D>(ka, pad, grid, block, lds, s);
    case 1: return launch_pad<NS, FK, 1, D>(ka, pad, grid, block, lds, s);
    case 2: return launch_pad<NS, FK, 2, D>(ka, pad, grid, block, lds, s);
    default: return launch_pad<NS, FK, 3, D>(ka, pad, grid, block, lds, s);
  }
}

template <int NS>
hipError_t launch_ns(const TopnKArgs& ka, bool fk, int vk, bool pad, int d, dim3 grid, dim3 block, uint32_t lds,
                     hipStream_t s) {
  if (d == 128) {
    if constexpr (NS <= 8) return launch_vk<NS, true, 128>(ka, vk, pad, grid, block, lds, s);
    return hipErrorInvalidValue;
  }
  return fk ? launch_vk<NS, true, 64>(ka, vk, pad, grid, block, lds, s)
            : launch_vk<NS, false, 64>(ka, vk, pad, grid, block, lds, s);
}

uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

}  // namespace

// Slots per lane the resident kernel is instantiated for (n <= 64 * slots).
static int resident_slots(int64_t n) {
  const int64_t s = (n + 63) / 64;
  if (s <= 1) return 1;
  if (s <= 2) return 2;
  if (s <= 4) return 4;
  if (s <= 8) return 8;
  if (s <= 12) return 12;
  if (s <= 16) return 16;
  return 0;
}

hipError_t launch_topn(const AttnParams& p, hipStream_t s) {
  if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
  const int NS = resident_slots(p.n);
  if (NS == 0 || (p.d == 128 && NS > 8)) return hipErrorInvalidValue;
  // head_dim 128 always takes the float-key path (exact for integer keys as well)
  const bool fused = p.xk != nullptr;
  // fused mean-centred codes come with scales: the float-key path
  const bool fk = p.alpha_q != nullptr || p.alpha_k != nullptr || p.bias != nullptr || p.brow != nullptr ||
                  p.d != 64 || (fused && p.mean);
  if (fused && p.mean && p.n > 256) return hipErrorInvalidValue;
  const int vk = p.v_kind;
  const int rowb = vk == 3 ? (int)p.d / 2 : (int)p.d * (vk == 0 ? 4 : (vk == 1 ? 2 : 1));
  TopnKArgs ka{};
  ka.qbits = p.qbits;
  ka.kbits = p.kbits;
  ka.aq = p.alpha_q;
  ka.ak = p.alpha_k;
  ka.xq = p.xq;
  ka.xk = p.xk;
  ka.qk_bf16 = p.qk_bf16;
  ka.mean = p.mean;
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
  ka.lcap = (int)((p.keep + 31) / 32 * 32);
  // query tiles of 64; when that leaves CUs idle (few heads), smaller tiles so that
  // about one workgroup per CU runs (each restages its head, cheap at these sizes)
  const int64_t bh_count = p.B * p.H;
  int64_t qt = kQTile;
  if (bh_count * ((p.n + kQTile - 1) / kQTile) < 256)
    qt = std::max<int64_t>(1, std::min<int64_t>(kQTile, (bh_count * p.n + 255) / 256));
  ka.qt = (int)qt;
  ka.tiles = (int)((p.n + qt - 1) / qt);
  ka.isd = (float)(1.0 / sqrt((double)p.d));
  ka.exp_c = (float)(2.0 * (double)ka.isd * 1.4426950408889634);
  uint32_t vbytes = align16((uint32_t)p.n * rowb);
  // fused: key code words and scales, the two means, and one tile's query code words and
  // scales; the mean-centred column sums use the V area (two sets of 256 x 8 float64)
  // before V is staged
  const uint32_t fused_bytes =
      fused ? align16((uint32_t)(p.n * (p.d / 32) * 4 + p.n * 4 + 2 * p.d * 4 + 64 * (p.d / 32) * 4 + 64 * 4)) : 0u;
  if (fused && p.mean) vbytes = std::max<uint32_t>(vbytes, 2u * 2048u * 8u);
  uint32_t bias_bytes = fk ? align16((uint32_t)(p.n + kQTile - 1) * 4u) : 0u;
  if (p.brow != nullptr) bias_bytes = align16((uint32_t)(bias2d_floats(p.gh, p.gw, p.cls) + p.n) * 4u);
  // as many waves as LDS allows (lists and candidate buffers are per wave)
  const uint32_t per_wave = (uint32_t)ka.lcap * (fk ? 8u : 12u) + (fk ? 64u * 8u : 256u);
  const uint32_t fixed = vbytes + bias_bytes + 4u * kMaxWaves + fused_bytes;
  int nw = kMaxWaves;
  while (nw > 1 && fixed + per_wave * nw > kLdsBytes) --nw;
  if (fixed + per_wave * nw > kLdsBytes) return hipErrorInvalidValue;
  ka.bias_off = vbytes;
  ka.list_off = vbytes + bias_bytes;
  ka.cand_off = ka.list_off + (uint32_t)ka.lcap * 8u * nw;
  ka.red_off = ka.cand_off + (fk ? 64u * 8u * nw : 0u);
  ka.keys_off = ka.red_off + 4u * kMaxWaves;
  ka.trash_off = ka.keys_off + (fk ? 0u : (uint32_t)ka.lcap * 4u * nw);
  ka.fused_off = ka.trash_off + (fk ? 0u : 256u * nw);
  const uint32_t lds = ka.fused_off + fused_bytes;
  if (fused && nw < 4) return hipErrorInvalidValue;  // (the column sums take 256 threads)
  // persistent workgroups: one per CU, each taking a contiguous run of units
  ka.units = (int)(p.B * p.H * ka.tiles);
  const int target = 256;
  ka.upw = (ka.units + target - 1) / target;
  const dim3 grid((unsigned)((ka.units + ka.upw - 1) / ka.upw));
  const dim3 block((unsigned)(64 * nw));
  const bool pad = p.n != (int64_t)NS * 64;  // padding keys exist in the last slots
  switch (NS) {
    case 1: return launch_ns<1>(ka, fk, vk, pad, (int)p.d, grid, block, lds, s);
    case 2: return launch_ns<2>(ka, fk, vk, pad, (int)p.d, grid, block, lds, s);
    case 4: return launch_ns<4>(ka, fk, vk, pad, (int)p.d, grid, block, lds, s);
    case 8: return launch_ns<8>(ka, fk, vk, pad, (int)p.d, grid, block, lds, s);
    case 12: return launch_ns<12>(ka, fk, vk, pad, (int)p.d, grid, block, lds, s);
    default: return launch_ns<16>(ka, fk, vk, pad, (int)p.d, grid, block, lds, s);
  }
}

}  // namespace had
