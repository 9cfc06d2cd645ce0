/*
 * had.h -- C ABI of the binarized-QK attention library (gfx950 / MI355X).
 *
 * The method (forward pass only):
 *   1. Q and K become {-1,+1} codes, bit-packed along head_dim:
 *      plain sign (Hamming Attention Distillation, abstract) or the
 *      mean-centred scaled sign alpha*sign(x - mu) of BinaryAttention
 *      (section 2.2, scaled binarized representation).  sign(0) = +1.
 *   2. Logit of query i and key j (BinaryAttention section 2.3, attention with
 *      bias; section 2.2, XNOR/popcount similarity):
 *         l = alpha_q[i]*alpha_k[j]*(d - 2*popcount(q XOR k)) / sqrt(d) + B[i][j]
 *   3. Optional per-query top-N (Hamming Attention Distillation, summary
 *      "main points"/"method": keep the N largest attention scores of each
 *      query), ties going to the lower key index.
 *   4. Softmax over the kept keys only, then A*V either in fp32
 *      (Hamming Attention Distillation keeps everything but K/Q full
 *      precision) or with A as uint8 at scale 1/255 and V as per-channel int8
 *      with integer accumulation (BinaryAttention section 2.4, mixed
 *      quantization).
 *
 * Conventions for every entry point
 *  - Tensors are contiguous, row-major, [B, H, n, .] (batch, head, token, .).
 *  - All tensor pointers are DEVICE pointers on the current HIP device.  The
 *    caller owns every buffer; the library never allocates or frees memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work and return; buffers must stay alive until the
 *    stream has executed it.  The library keeps no state between calls and may
 *    be called from several host threads.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error status nothing is launched and no output is touched.  Faults that
 *    happen on the device surface at the caller's next synchronisation.
 *  - d must be 32, 64 or 128 (bits per token: d/32 uint32 words) for packing;
 *    the attention entry points take d = 64 or d = 128.
 *  - Relative-position bias: `bias_table` is float32 [H, 2n-1] and
 *    B[i][j] = bias_table[h][j - i + n - 1]; NULL means B = 0.
 *  - alpha pointers: float32 [B, H, n]; NULL means alpha = 1.
 *  - Inputs must be finite (no NaN/Inf); a NaN input gets code +1.
 */
#ifndef HAD_H
#define HAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HAD_ABI_VERSION 1

/* status codes */
#define HAD_OK 0
#define HAD_ERR_INVALID_ARG 1 /* NULL required pointer, size <= 0, top_n < 1, unknown enum */
#define HAD_ERR_UNSUPPORTED 2 /* a size outside what the kernels are built for */
#define HAD_ERR_WORKSPACE 3   /* workspace NULL or smaller than had_workspace_bytes() */
#define HAD_ERR_HIP 4         /* the HIP runtime reported an error at launch */

/* element types of x / v */
#define HAD_F32 0
#define HAD_BF16 1

/* binarization modes */
#define HAD_SIGN 0      /* code = sign(x); alpha = 1 */
#define HAD_MEAN_SIGN 1 /* code = sign(x - mu); alpha = mean_c |x - mu| */

/* A*V modes */
#define HAD_AV_F32 0 /* fp32 probabilities times V, fp32 accumulation */
#define HAD_AV_Q8 1  /* uint8 A (scale 1/255) times per-channel int8 V, int32 accumulation */
#define HAD_AV_Q4 2  /* as HAD_AV_Q8 with 4-bit V: 7 levels each side of zero (scale max|V|/7) */

/* Largest sizes the kernels accept.  top_n itself is unbounded: min(top_n, n) keys
 * are kept, so the kept set never exceeds HAD_MAX_TOPN = HAD_MAX_N. */
#define HAD_MAX_N 65536
#define HAD_MAX_TOPN 65536

int had_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* had_status_str(int status);

/*
 * Bytes of device workspace any entry point needs for these sizes (a single
 * buffer of this size serves had_pack, had_pack_qk, had_attention_topn and
 * binattn_dense_q8).  Multiple of 256.  Contents need not be initialised.
 */
size_t had_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d);

/* Regions of the workspace that hold results after a quantized attention call. */
#define HAD_WS_VQ 0     /* int8 V, [B,H,n,d], one byte per element */
#define HAD_WS_VSCALE 1 /* float32 per-channel V scales, [B,H,d] */

/*
 * Byte offset and size of region `region` (HAD_WS_VQ or HAD_WS_VSCALE) inside a
 * workspace of had_workspace_bytes(B,H,n,d) bytes, so that a caller can read the
 * integer V and its scales that a quantized attention call leaves there.  Writes
 * *offset and *bytes and returns HAD_OK; HAD_ERR_INVALID_ARG for an unknown
 * region, NULL outputs or sizes had_workspace_bytes rejects.  Host-only.
 */
int had_workspace_region(int64_t B, int64_t H, int64_t n, int64_t d, int region, size_t* offset, size_t* bytes);

/*
 * had_pack -- binarize and bit-pack one of Q or K.
 * (Hamming Attention Distillation, abstract: {-1,+1} keys and queries;
 *  BinaryAttention section 2.2: x~ = alpha * sign(x - mu).)
 *
 *  x        [B,H,n,d] of x_dtype (HAD_F32 or HAD_BF16)
 *  mode     HAD_SIGN or HAD_MEAN_SIGN
 *  bits     out uint32 [B,H,n,d/32]: bit (c%32) of word c/32 is 1 iff the code
 *           of channel c is -1, i.e. iff y < 0 where y = x (SIGN) or
 *           y = float32(x - mu) (MEAN_SIGN).
 *  alpha    out float32 [B,H,n]: MEAN_SIGN: float32(sum_c |y| / d) with the sum
 *           in float64; SIGN: filled with 1.0f.  Required for MEAN_SIGN,
 *           may be NULL for SIGN.
 *  mu       out float32 [B,H,d]: MEAN_SIGN: float32(sum_i x / n), sum in
 *           float64, mean over tokens per (batch, head, channel); SIGN: 0.
 *           Required for MEAN_SIGN, may be NULL for SIGN.
 *  workspace, workspace_bytes: device scratch of at least
 *           had_workspace_bytes(B,H,n,d) bytes (MEAN_SIGN only; may be NULL for SIGN).
 */
int had_pack(const void* x, int x_dtype, int64_t B, int64_t H, int64_t n, int64_t d, int mode,
             uint32_t* bits, float* alpha, float* mu, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * had_pack_qk -- binarize and bit-pack Q and K of one layer in one set of launches
 * (the same passages as had_pack).  Each output is exactly what had_pack gives for
 * that tensor alone; Q and K share x_dtype, sizes and mode.
 *
 *  q, k              [B,H,n,d] of x_dtype
 *  qbits, kbits      out uint32 [B,H,n,d/32]
 *  alpha_q, alpha_k  out float32 [B,H,n] (required for MEAN_SIGN, may be NULL for SIGN)
 *  mu_q, mu_k        out float32 [B,H,d] (required for MEAN_SIGN, may be NULL for SIGN)
 *  workspace, workspace_bytes: as for had_pack (the layout holds the column-sum
 *           partials of both tensors).
 * Errors: as had_pack.  Buffers are caller-owned; nothing is allocated.
 */
int had_pack_qk(const void* q, const void* k, int x_dtype, int64_t B, int64_t H, int64_t n, int64_t d, int mode,
                uint32_t* qbits, uint32_t* kbits, float* alpha_q, float* alpha_k, float* mu_q, float* mu_k,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * had_attention_topn -- attention over each query's top-N keys.
 * (Hamming Attention Distillation, summary "main points"/"method": per query
 *  keep the top N attention scores, prune the rest before softmax and V
 *  accumulation; BinaryAttention sections 2.3-2.4 for the bias and the
 *  quantized A*V.)
 *
 *  qbits, kbits   uint32 [B,H,n,d/32] from had_pack
 *  alpha_q, alpha_k  float32 [B,H,n] or NULL (alpha = 1)
 *  bias_table     float32 [H,2n-1] or NULL (B = 0)
 *  v              [B,H,n,d] of v_dtype (HAD_F32 or HAD_BF16)
 *  top_n          N >= 1; N >= n keeps every key (dense softmax).  Any N at any
 *                 n: short sequences keep a head on chip; long ones stream keys
 *                 with a bounded candidate buffer, or, for kept sets beyond it,
 *                 find the N-th largest logit first (radix selection over the
 *                 keys) and then gather the kept keys
 *  av_mode        HAD_AV_F32, HAD_AV_Q8 or HAD_AV_Q4
 *  out            out float32 [B,H,n,d]
 *  idx_out        optional out int32 [B,H,n,min(N,n)]: kept key indices of
 *                 each query in ascending order; NULL to skip
 *  workspace      >= had_workspace_bytes(B,H,n,d) bytes (HAD_AV_Q8 and
 *                 HAD_AV_Q4; may be NULL for HAD_AV_F32).  On return (after
 *                 the stream has run) it holds the integer V and its
 *                 per-channel scales: HAD_AV_Q8 one int8 per element;
 *                 HAD_AV_Q4 two 4-bit two's-complement codes per byte
 *                 (byte b of a row: channel 2b in the low nibble, channel
 *                 2b + 1 in the high nibble), in the same region.
 *
 *  Logit, in float32 with each operation rounded as written:
 *      t = alpha_q*alpha_k;  u = t*(d-2h);  v = u*float(1/sqrt(d));  l = v + B
 *  The kept set is the N largest l, ties to the lower key index; it is exact.
 *  Softmax in float32 over the kept set.  HAD_AV_Q8: scale_c = max_j|V[j][c]|/127
 *  over all n tokens, Vq = clamp(rint(V/scale_c), -127, 127),
 *  A_q = clamp(rint(255 p), 0, 255), O = float(sum A_q*Vq) * scale_c / 255.
 *  HAD_AV_Q4 (the 4-bit V that BinaryAttention's conclusion names as the next
 *  step): the same with 7 in place of 127, the codes stored two per byte; the
 *  kernels widen them to bytes for the 8-bit dot products (gfx950 has no
 *  4-bit integer matrix instruction).
 */
int had_attention_topn(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q,
                       const float* alpha_k, const float* bias_table, const void* v, int v_dtype,
                       int64_t B, int64_t H, int64_t n, int64_t d, int64_t top_n, int av_mode,
                       float* out, int32_t* idx_out, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * binattn_dense_q8 -- BinaryAttention forward: dense softmax over all keys,
 * uint8 A (scale 1/255) times per-channel int8 V with int32 accumulation
 * (BinaryAttention section 2.4: O = dequant(matmul(quant_u8(A), quant_i8(V)))).
 * Same arguments and arithmetic as had_attention_topn with top_n = n and
 * av_mode = HAD_AV_Q8; the contraction runs on int8 matrix cores.  Any n up to
 * HAD_MAX_N: up to 256 tokens one workgroup keeps a head on chip; beyond, keys
 * stream through on-chip memory in tiles, in two passes (row maximum and
 * normaliser, then the quantized product).
 * workspace is required (>= had_workspace_bytes(B,H,n,d)).
 */
int binattn_dense_q8(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q,
                     const float* alpha_k, const float* bias_table, const void* v, int v_dtype,
                     int64_t B, int64_t H, int64_t n, int64_t d, float* out, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * had_attention_topn_2d, binattn_dense_q8_2d -- had_attention_topn and
 * binattn_dense_q8 with a two-dimensional decomposable relative-position bias in
 * place of bias_table (BinaryAttention section 4.4: a bias that is a sum of
 * terms keeps the bias memory negligible at high resolution; section 2.3 for the
 * bias in the logit).  The n tokens are an optional class token followed by a
 * grid_h x grid_w grid of patches in row-major order (n = grid_h*grid_w, plus 1
 * with a class token).  For patches i = (r_i, c_i) and j = (r_j, c_j):
 *     B[i][j] = row_table[h][r_j - r_i + grid_h - 1] + col_table[h][c_j - c_i + grid_w - 1]
 * (one float32 addition); with cls_table (float32 [H,3]) the class token is
 * token 0 and B = cls_table[h][0] for class -> patch, [1] for patch -> class,
 * [2] for class -> class.  cls_table NULL: no class token.
 *
 *  row_table   float32 [H, 2*grid_h-1]     col_table   float32 [H, 2*grid_w-1]
 *
 * All other arguments, the arithmetic and the errors as the 1-D entry points.
 * HAD_ERR_INVALID_ARG: NULL table, grid sizes < 1 or n inconsistent with the grid;
 * HAD_ERR_UNSUPPORTED: grid_h or grid_w above 13000, or tables of
 * (2*grid_h-1)+(2*grid_w-1) floats (5*(grid_h+grid_w)-2 with a class token) above
 * what the kernel keeps on chip beside its key tiles: 1536 for top-N above the
 * resident limit, 4096 for the dense entry point above 256
 * tokens.
 */
int had_attention_topn_2d(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q,
                          const float* alpha_k, const float* row_table, const float* col_table,
                          const float* cls_table, int64_t grid_h, int64_t grid_w, const void* v, int v_dtype,
                          int64_t B, int64_t H, int64_t n, int64_t d, int64_t top_n, int av_mode, float* out,
                          int32_t* idx_out, void* workspace, size_t workspace_bytes, void* stream);
int binattn_dense_q8_2d(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q,
                        const float* alpha_k, const float* row_table, const float* col_table,
                        const float* cls_table, int64_t grid_h, int64_t grid_w, const void* v, int v_dtype,
                        int64_t B, int64_t H, int64_t n, int64_t d, float* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * had_attention_topn_fused -- had_pack_qk followed by had_attention_topn (fp32
 * A*V) in one launch, for sequences one workgroup holds on chip (Hamming
 * Attention Distillation, abstract and summary "method": {-1,+1} keys and
 * queries, top-N per query; BinaryAttention section 2.2 for the mean-centred
 * codes and section 2.3 for the bias).  A workgroup binarizes the keys of its head
 * (and, mean-centred, takes the means of Q and K) on chip and each query's code
 * as it goes, with had_pack's arithmetic and summation order, then runs the
 * top-N attention on them.
 *
 *  q, k        [B,H,n,d] of qk_dtype (HAD_F32 or HAD_BF16)
 *  mode        HAD_SIGN or HAD_MEAN_SIGN (as had_pack)
 *  bias_table  float32 [H,2n-1] or NULL (B = 0)
 *  v           [B,H,n,d] of v_dtype (HAD_F32 or HAD_BF16)
 *  top_n       N >= 1 (N >= n keeps every key)
 *  out         out float32 [B,H,n,d]
 *  idx_out     optional out int32 [B,H,n,min(N,n)], ascending key index
 *
 * The kept index sets are those of had_pack_qk + had_attention_topn on the same
 * inputs; the outputs are the same bits where that pair runs the resident kernel
 * (fp32 V, mean-centred codes or head_dim 128) and within the fp32 tolerance
 * otherwise.  No workspace and no intermediate tensor.  n up to 512 (fp32 V) or
 * 1024 (bf16 V), half that at d = 128, and at most 256 for HAD_MEAN_SIGN; d = 64
 * or 128; else HAD_ERR_UNSUPPORTED.  Other errors as had_pack and
 * had_attention_topn.
 */
int had_attention_topn_fused(const void* q, const void* k, int qk_dtype, int mode, const float* bias_table,
                             const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d, int64_t top_n,
                             float* out, int32_t* idx_out, void* stream);

/*
 * binattn_dense_q8_fused -- binattn_dense_q8 with the binarization and the V
 * quantization in the same launch, for short sequences (BinaryAttention
 * section 2.2 codes and scales, section 2.3 logits, section 2.4 quantized A*V).
 * One workgroup per (batch, head) binarizes that head's Q and K and quantizes
 * its V in on-chip memory, then runs the dense q8 attention on them.
 *
 *  q, k        [B,H,n,d] of qk_dtype (HAD_F32 or HAD_BF16)
 *  mode        HAD_SIGN or HAD_MEAN_SIGN (as had_pack)
 *  bias_table  float32 [H,2n-1] or NULL (B = 0)
 *  v           [B,H,n,d] of v_dtype (HAD_F32 or HAD_BF16)
 *  out         out float32 [B,H,n,d]
 *
 * The result is bit-identical to had_pack_qk followed by binattn_dense_q8 on
 * the same inputs (same arithmetic, summation order and rounding).  No
 * workspace and no intermediate tensor: codes, alpha, mu and the int8 V are not
 * returned.  n <= 256 and d = 64 or 128, else HAD_ERR_UNSUPPORTED; other errors
 * as had_pack and binattn_dense_q8.
 */
int binattn_dense_q8_fused(const void* q, const void* k, int qk_dtype, int mode, const float* bias_table,
                           const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d, float* out,
                           void* stream);

/*
 * binattn_dense_q8_noalloc -- binattn_dense_q8 for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, arithmetic and results as
 * binattn_dense_q8, without the workspace: the integer V, its scales and the
 * partial maxima live in a static device array of HAD_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.  No
 * call allocates or frees memory.
 *
 * Sizes whose workspace (had_workspace_bytes(B,H,n,d)) exceeds
 * HAD_NOALLOC_SCRATCH_BYTES return HAD_ERR_UNSUPPORTED before anything is
 * enqueued; other errors as binattn_dense_q8.  All calls on one GPU share that
 * GPU's array: calls that overlap in time on one GPU (on different streams or
 * host threads) race on it and must be ordered by the caller.  The array keeps
 * what the last call left; no call reads anything before writing it.
 */
#define HAD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int binattn_dense_q8_noalloc(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q,
                             const float* alpha_k, const float* bias_table, const void* v, int v_dtype,
                             int64_t B, int64_t H, int64_t n, int64_t d, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HAD_H */
