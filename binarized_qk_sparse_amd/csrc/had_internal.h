// Host-side declarations shared by the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace had {

// ---- packing (pack.hip)
struct PackSet {
  const void* x;
  uint32_t* bits;
  float* alpha;
  float* mu;
  double* partial;  // MEAN_SIGN: [BH, chunks, d] float64 column sums
};
struct PackParams {
  int x_dtype;  // HAD_F32 / HAD_BF16
  int64_t BH, n, d;
  int mode;   // HAD_SIGN / HAD_MEAN_SIGN
  int count;  // tensors packed by the launches: 1 (had_pack) or 2 (had_pack_qk)
  PackSet set[2];
};
constexpr int kPackChunk = 256;  // tokens per column-sum chunk
inline int64_t pack_chunks(int64_t n) { return (n + kPackChunk - 1) / kPackChunk; }
hipError_t launch_pack(const PackParams& p, hipStream_t s);

// ---- V quantization (vquant.hip)
struct VQuantParams {
  const void* v;
  int v_dtype;
  int64_t BH, n, d;
  float* vmax_partial;  // [BH, chunks, d]
  float* vscale;        // [BH, d]
  int8_t* vq;           // [BH, n, d] int8, or [BH, n, d/2] bytes of two 4-bit codes (levels 7)
  int levels;           // 127 (int8) or 7 (4-bit values)
};
constexpr int kVqChunk = 256;
inline int64_t vq_chunks(int64_t n) { return (n + kVqChunk - 1) / kVqChunk; }
hipError_t launch_vquant(const VQuantParams& p, hipStream_t s);

// ---- attention (topn.hip, dense_q8.hip)
struct AttnParams {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const float* alpha_q;
  const float* alpha_k;
  const float* bias;
  const void* v;  // f32 / bf16 V (AV_F32), int8 Vq (AV_Q8) or packed 4-bit Vq (AV_Q4)
  int v_kind;     // 0 f32, 1 bf16, 2 int8 codes, 3 4-bit codes two per byte (quantized)
  const float* vscale;
  int64_t B, H, n, d;
  int64_t keep;  // min(top_n, n)
  float* out;
  int32_t* idx;
  // two-dimensional decomposable bias (in place of `bias`, which is then NULL):
  // row and column offset tables over a gh x gw patch grid that follows `cls`
  // (0 or 1) class tokens, and the class token's three values; brow == NULL: none
  const float* brow;
  const float* bcol;
  const float* bcls;
  int gh, gw, cls;
  // fused top-N (resident kernel): raw Q and K (fp32 or bf16) binarized on chip in
  // place of qbits/kbits/alpha (xk == NULL: not fused)
  const void* xq;
  const void* xk;
  int qk_bf16, mean;
};
// floats of the staged two-dimensional bias tables (rows and columns with the
// class token's values folded in; see had_device.hpp)
__host__ __device__ inline int64_t bias2d_floats(int64_t gh, int64_t gw, int64_t cls) {
  return cls ? (5 * gh - 1) + (5 * gw - 1) : (2 * gh - 1) + (2 * gw - 1);
}
hipError_t launch_topn(const AttnParams& p, hipStream_t s);
// largest n the resident top-N kernel takes for V of kind v_kind (0 f32, 1 bf16, 2 int8, 3 int4)
int64_t topn_resident_max_n(int v_kind, int64_t d);
bool topn_mfma_supported(const AttnParams& p);
hipError_t launch_topn_mfma(const AttnParams& p, hipStream_t s);
hipError_t launch_topn_stream(const AttnParams& p, hipStream_t s);
// whether the streaming kernel takes n keys, kept sets of `keep` and two-dimensional
// bias tables of `tab` floats (0: none)
bool topn_stream_takes(int64_t n, int64_t keep, int64_t tab);
// top-N above the resident limit with more kept keys than the streaming kernel
// buffers (topn_wide.hip): threshold by radix selection, then the kept keys
hipError_t launch_topn_wide(const AttnParams& p, hipStream_t s);
int64_t topn_wide_bias2d_max();
hipError_t launch_dense_q8(const AttnParams& p, hipStream_t s);
int64_t dense_q8_max_n();
// dense q8 attention for n above dense_q8_max_n() (dense_long.hip): keys streamed in tiles
hipError_t launch_dense_long(const AttnParams& p, hipStream_t s);
int64_t dense_long_bias2d_max();

// ---- binarize + quantize + dense q8 attention in one launch (dense_q8.hip)
struct DenseFusedParams {
  const void* q;
  const void* k;
  const void* v;
  int qk_dtype, v_dtype;  // HAD_F32 / HAD_BF16
  int mode;               // HAD_SIGN / HAD_MEAN_SIGN
  const float* bias;
  int64_t B, H, n, d;
  float* out;
};
hipError_t launch_dense_q8_fused(const DenseFusedParams& p, hipStream_t s);

// binattn_dense_q8 with its checks and dispatch, for entry points that supply the
// workspace themselves (`fn` names the caller in debug messages).
int dense_q8_entry(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                   const float* bias_table, const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                   float* out, void* workspace, size_t workspace_bytes, void* stream, const char* fn);
// The argument checks of binattn_dense_q8 short of the workspace (no HIP call).
int dense_q8_check(const uint32_t* qbits, const uint32_t* kbits, const void* v, int v_dtype, int64_t B, int64_t H,
                   int64_t n, int64_t d, float* out, const char* fn);
// Returns `status`, printing `why` under HAD_DEBUG.
int report(int status, const char* fn, const char* why);

// Device scratch layout inside the caller's workspace.
struct WorkspaceLayout {
  size_t pack_partial;  // offset of double[BH, pack_chunks, d]
  size_t pack_partial2;  // offset of the second tensor's (had_pack_qk)
  size_t vq;            // offset of int8[BH, n, d]
  size_t vscale;        // offset of float[BH, d]
  size_t vmax_partial;  // offset of float[BH, vq_chunks, d]
  size_t total;
};
WorkspaceLayout workspace_layout(int64_t B, int64_t H, int64_t n, int64_t d);

}  // namespace had
