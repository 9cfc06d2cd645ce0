/*
 * CPU oracle for binarized-QK attention.  TEST INFRASTRUCTURE ONLY: it is
 * called by the tests, by the smoke check and by the CPU-baseline leg of the
 * benchmark, never by the product path.  It shares no code, header or
 * constant generator with the GPU library.
 *
 * Plain C99, no intrinsics, built with -O2 -ffp-contract=off so that every
 * float expression below is rounded exactly as written.  OpenMP only spreads
 * independent query rows over threads.
 *
 * Sources (titles of the pages the method is described on):
 *  [HAD]  "Hamming Attention Distillation: Binarizing Keys and Queries for
 *         Efficient Long-Context Transformers": abstract (K/Q turned into
 *         {-1,+1} vectors, dot product replaced by Hamming distance, attention
 *         matrix sparsified), AI summary "main points" and "method" (per-query
 *         top-N of the attention scores, N schedule; everything other than K/Q
 *         stays full precision).
 *  [BA]   "BinaryAttention: One-Bit QK-Attention for Vision and Diffusion
 *         Transformers" (blog write-up): section 2.2 (scaled binarization
 *         alpha*sign(x-mu); XNOR+popcount similarity), section 2.3 (attention
 *         with additive bias B, Softmax(QK^T/sqrt(d)+B)V; relative position
 *         bias), section 2.4 (A -> uint8 with scale 1/255, V -> per-channel
 *         int8, O = dequant(matmul(quant_u8(A), quant_i8(V)))).
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *  - sign(0) = +1; a code bit is 1 exactly when the value is < 0.
 *  - mu is the per-(batch, head, channel) mean over tokens; alpha is the
 *    per-token mean of |x - mu| over channels.
 *  - the bias is a per-head table over 2n-1 offsets, B[i][j] = T[j - i + n - 1].
 *  - the logit is formed in float32 in the order
 *        t = aq*ak;  u = t*dot;  v = u*s;  l = v + T,   s = float(1/sqrt(d)),
 *    because the top-N decision is taken on it and the kernel takes it in
 *    float32 too.
 *  - top-N keeps the N largest logits, ties going to the lower key index;
 *    N >= n keeps every key (dense attention).
 *  - softmax runs in float64 over the kept set only.
 *  - quantization rounds to nearest even; V scale = max|V[:,c]| / 127 per
 *    (batch, head, channel); A_q = clamp(rint(255 p), 0, 255).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_SIGN 0
#define OR_MEAN_SIGN 1
#define OR_AV_F32 0
#define OR_AV_Q8 1
#define OR_AV_Q4 2

/* Number of threads the OpenMP loops below use. */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int t) {
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}

/* ---------------------------------------------------------------- binarize
 * [HAD] abstract: keys and queries become {-1,+1} vectors (plain sign).
 * [BA] 2.2: Q~ = alpha_Q * sign(Q - mu_Q), K~ = alpha_K * sign(K - mu_K).
 *
 * x      float32 [B,H,n,d] (bf16 inputs are widened exactly before the call)
 * bits   uint32  [B,H,n,d/32]; bit (c%32) of word c/32 is 1 iff code is -1
 * alpha  float32 [B,H,n] (MEAN_SIGN: mean |x-mu| over channels; SIGN: 1)
 * mu     float32 [B,H,d] (MEAN_SIGN: mean over tokens; SIGN: 0)
 * alpha/mu may be NULL for SIGN.
 */
void oracle_pack(const float* x, int64_t B, int64_t H, int64_t n, int64_t d, int mode,
                 uint32_t* bits, float* alpha, float* mu) {
    const int64_t W = d / 32;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const float* xs = x + bh * n * d;
        float* m = mu ? mu + bh * d : NULL;
        float* mloc = (float*)malloc((size_t)d * sizeof(float));
        for (int64_t c = 0; c < d; ++c) {
            float mc = 0.0f;
            if (mode == OR_MEAN_SIGN) {
                double s = 0.0;
                for (int64_t i = 0; i < n; ++i) s += (double)xs[i * d + c];
                mc = (float)(s / (double)n);
            }
            mloc[c] = mc;
            if (m) m[c] = mc;
        }
        for (int64_t i = 0; i < n; ++i) {
            uint32_t* row = bits + (bh * n + i) * W;
            for (int64_t w = 0; w < W; ++w) row[w] = 0u;
            double asum = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                float y = xs[i * d + c];
                if (mode == OR_MEAN_SIGN) y = y - mloc[c];
                if (y < 0.0f) row[c / 32] |= (uint32_t)1u << (c % 32);
                asum += fabs((double)y);
            }
            if (alpha) alpha[bh * n + i] = (mode == OR_MEAN_SIGN) ? (float)(asum / (double)d) : 1.0f;
        }
        free(mloc);
    }
}

/* Number of set bits, one bit at a time. */
static int count_ones(uint32_t w) {
    int c = 0;
    for (int b = 0; b < 32; ++b) c += (int)((w >> b) & 1u);
    return c;
}

/* [HAD] abstract; [BA] 2.2: for +-1 codes the dot product is
 * d - 2 * (number of positions where the codes differ). */
static int32_t hamming(const uint32_t* a, const uint32_t* b, int64_t W) {
    int32_t h = 0;
    for (int64_t w = 0; w < W; ++w) h += count_ones(a[w] ^ b[w]);
    return h;
}

/* float(1/sqrt(d)): the 1/sqrt(d) factor of [BA] 2.3, rounded once. */
static float inv_sqrt_d(int64_t d) { return (float)(1.0 / sqrt((double)d)); }

/* Decomposable two-dimensional relative-position bias ([BA] 4.4: a sum of
 * biases that keeps the bias memory negligible; [BA] 2.3 for the bias itself).
 * Tokens are an optional leading class token (cls = 1) followed by a gh x gw
 * grid of patches in row-major order.  For two patches the bias is a row term
 * plus a column term, each a per-head table over the signed offsets:
 *     R[h][r_j - r_i + gh - 1] + C[h][c_j - c_i + gw - 1]    (float32 sum)
 * and a pair involving the class token takes one of three per-head values
 * X[h][0] (class -> patch), X[h][1] (patch -> class), X[h][2] (class -> class). */
typedef struct {
    const float* R;   /* [H, 2 gh - 1] */
    const float* C;   /* [H, 2 gw - 1] */
    const float* X;   /* [H, 3] (cls = 1 only) */
    int64_t gh, gw, cls;
} bias2d_t;

static float bias2d_value(const bias2d_t* b, int64_t h, int64_t i, int64_t j) {
    const int64_t ci = i < b->cls, cj = j < b->cls;
    if (ci && cj) return b->X[h * 3 + 2];
    if (ci) return b->X[h * 3 + 0];
    if (cj) return b->X[h * 3 + 1];
    const int64_t pi = i - b->cls, pj = j - b->cls;
    const int64_t ri = pi / b->gw, cli = pi % b->gw, rj = pj / b->gw, clj = pj % b->gw;
    return b->R[h * (2 * b->gh - 1) + (rj - ri + b->gh - 1)] + b->C[h * (2 * b->gw - 1) + (clj - cli + b->gw - 1)];
}

/* The logit of query i, key j ([BA] 2.3 with the scaled codes of [BA] 2.2):
 * bias from the 1-D offset table T, the 2-D decomposable form b2, or none. */
static float logit(const uint32_t* qb, const uint32_t* kb, const float* aq, const float* ak,
                   const float* T, const bias2d_t* b2, int64_t n, int64_t d, int64_t bh, int64_t h_idx, int64_t i,
                   int64_t j, int32_t* ham_out) {
    const int64_t W = d / 32;
    int32_t h = hamming(qb + (bh * n + i) * W, kb + (bh * n + j) * W, W);
    int32_t dot = (int32_t)d - 2 * h;
    float t = (aq ? aq[bh * n + i] : 1.0f) * (ak ? ak[bh * n + j] : 1.0f);
    float u = t * (float)dot;
    float v = u * inv_sqrt_d(d);
    float l = v;
    if (b2) l = v + bias2d_value(b2, h_idx, i, j);
    else if (T) l = v + T[h_idx * (2 * n - 1) + (j - i + n - 1)];
    if (ham_out) *ham_out = h;
    return l;
}

/* Full Hamming-distance and logit matrices, [B,H,n,n] each (small cases). */
void oracle_logits(const uint32_t* qb, const uint32_t* kb, const float* aq, const float* ak,
                   const float* T, const float* R2, const float* C2, const float* X2, int64_t gh, int64_t gw,
                   int64_t cls, int64_t B, int64_t H, int64_t n, int64_t d, int32_t* ham, float* logits) {
    const bias2d_t b2v = {R2, C2, X2, gh, gw, cls};
    const bias2d_t* b2 = R2 ? &b2v : NULL;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            int64_t bh = b * H + h;
            for (int64_t i = 0; i < n; ++i)
                for (int64_t j = 0; j < n; ++j) {
                    int32_t hd;
                    float l = logit(qb, kb, aq, ak, T, b2, n, d, bh, h, i, j, &hd);
                    if (ham) ham[(bh * n + i) * n + j] = hd;
                    if (logits) logits[(bh * n + i) * n + j] = l;
                }
        }
}

/* --------------------------------------------------------- V quantization
 * [BA] 2.4: per-channel integer quantization of V with `levels` levels each
 * side of zero: 127 (int8, the pages' design) or 7 (the 4-bit V that the pages
 * name as the next step).
 * scale[c] = max_j |V[j][c]| / levels (float32 division);
 * Vq = clamp(rint(V/scale), -levels, levels), 0 where the scale is 0.
 */
void oracle_vquant_levels(const float* v, int64_t B, int64_t H, int64_t n, int64_t d, int levels, int8_t* vq,
                          float* scale) {
    const float lv = (float)levels;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const float* vs = v + bh * n * d;
        for (int64_t c = 0; c < d; ++c) {
            float mx = 0.0f;
            for (int64_t j = 0; j < n; ++j) {
                float a = fabsf(vs[j * d + c]);
                if (a > mx) mx = a;
            }
            float sc = mx / lv;
            scale[bh * d + c] = sc;
            for (int64_t j = 0; j < n; ++j) {
                int32_t q = 0;
                if (sc > 0.0f) {
                    float r = rintf(vs[j * d + c] / sc);
                    if (r > lv) r = lv;
                    if (r < -lv) r = -lv;
                    q = (int32_t)r;
                }
                vq[(bh * n + j) * d + c] = (int8_t)q;
            }
        }
    }
}

void oracle_vquant(const float* v, int64_t B, int64_t H, int64_t n, int64_t d, int8_t* vq, float* scale) {
    oracle_vquant_levels(v, B, H, n, d, 127, vq, scale);
}

typedef struct {
    float l;
    int32_t j;
} scored_t;

/* Larger logit first; equal logits: lower key index first. */
static int by_logit_then_index(const void* pa, const void* pb) {
    const scored_t* a = (const scored_t*)pa;
    const scored_t* b = (const scored_t*)pb;
    if (a->l > b->l) return -1;
    if (a->l < b->l) return 1;
    return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int by_index(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/* ---------------------------------------------------------------- attention
 * One query row r = (b*H + h)*n + i at a time:
 *   logits over all keys -> keep the top-N ([HAD] summary: top N attention
 *   scores per query) -> softmax over the kept set ([BA] 2.3) -> A*V in
 *   float64 (av_mode F32, [HAD]: full-precision A*V) or as uint8 A times
 *   per-channel integer V with integer accumulation (av_mode Q8 or Q4,
 *   [BA] 2.4; the two differ only in the quantization of V done beforehand).
 *
 * rows     flat query-row indices to compute (NULL: all B*H*n rows in order)
 * out      float32 [nrows, d]
 * idx      int32 [nrows, min(N,n)] kept key indices in ascending order, or NULL
 * aq8      int32 [nrows, min(N,n)] A_q of those keys (Q8/Q4 only), or NULL
 * vq/vscale  int8 [B,H,n,d] and float32 [B,H,d] from oracle_vquant_levels (Q8/Q4 only)
 * Returns 0, or -1 if an int32 accumulator would overflow (Q8).
 */
int oracle_attention(const uint32_t* qb, const uint32_t* kb, const float* aq, const float* ak,
                     const float* T, const float* R2, const float* C2, const float* X2, int64_t gh, int64_t gw,
                     int64_t cls, const float* v, const int8_t* vq, const float* vscale,
                     int64_t B, int64_t H, int64_t n, int64_t d, int64_t top_n, int av_mode,
                     const int64_t* rows, int64_t nrows, float* out, int32_t* idx, int32_t* aq8) {
    const bias2d_t b2v = {R2, C2, X2, gh, gw, cls};
    const bias2d_t* b2 = R2 ? &b2v : NULL;
    const int64_t keep = top_n < n ? top_n : n;
    int failed = 0;
    if (rows == NULL) nrows = B * H * n;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : failed)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t bh = flat / n, i = flat % n, h = bh % H;
        scored_t* s = (scored_t*)malloc((size_t)n * sizeof(scored_t));
        int32_t* kept = (int32_t*)malloc((size_t)keep * sizeof(int32_t));
        double* p = (double*)malloc((size_t)n * sizeof(double));
        for (int64_t j = 0; j < n; ++j) {
            s[j].l = logit(qb, kb, aq, ak, T, b2, n, d, bh, h, i, j, NULL);
            s[j].j = (int32_t)j;
        }
        qsort(s, (size_t)n, sizeof(scored_t), by_logit_then_index);
        /* softmax over the kept set; s[0] holds the largest logit */
        double z = 0.0;
        for (int64_t t = 0; t < keep; ++t) z += exp((double)s[t].l - (double)s[0].l);
        for (int64_t j = 0; j < n; ++j) p[j] = 0.0;
        for (int64_t t = 0; t < keep; ++t) {
            p[s[t].j] = exp((double)s[t].l - (double)s[0].l) / z;
            kept[t] = s[t].j;
        }
        qsort(kept, (size_t)keep, sizeof(int32_t), by_index);
        float* o = out + r * d;
        if (av_mode == OR_AV_F32) {
            for (int64_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t t = 0; t < keep; ++t) {
                    int64_t j = kept[t];
                    acc += p[j] * (double)v[(bh * n + j) * d + c];
                }
                o[c] = (float)acc;
            }
        } else {
            for (int64_t c = 0; c < d; ++c) {
                int64_t acc = 0;
                for (int64_t t = 0; t < keep; ++t) {
                    int64_t j = kept[t];
                    double a = rint(255.0 * p[j]);
                    if (a < 0.0) a = 0.0;
                    if (a > 255.0) a = 255.0;
                    acc += (int64_t)a * (int64_t)vq[(bh * n + j) * d + c];
                }
                if (acc > INT32_MAX || acc < INT32_MIN) failed |= 1;
                float sc = vscale[bh * d + c];
                o[c] = ((float)acc * sc) / 255.0f;
            }
        }
        for (int64_t t = 0; t < keep; ++t) {
            if (idx) idx[r * keep + t] = kept[t];
            if (aq8) {
                double a = rint(255.0 * p[kept[t]]);
                aq8[r * keep + t] = (int32_t)(a < 0.0 ? 0.0 : (a > 255.0 ? 255.0 : a));
            }
        }
        free(s);
        free(kept);
        free(p);
    }
    return failed ? -1 : 0;
}
