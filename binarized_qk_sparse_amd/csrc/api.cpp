// C ABI of the binarized-QK attention library: argument validation,
// workspace layout and kernel dispatch.  Every check runs before anything is
// enqueued, so an error status means nothing was launched.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/had.h"
#include "had_internal.h"

namespace had {

static size_t align256(size_t x) { return (x + 255u) & ~(size_t)255u; }

WorkspaceLayout workspace_layout(int64_t B, int64_t H, int64_t n, int64_t d) {
  WorkspaceLayout w{};
  const int64_t BH = B * H;
  size_t off = 0;
  w.pack_partial = off;
  off = align256(off + sizeof(double) * (size_t)(BH * pack_chunks(n) * d));
  w.vq = off;
  off = align256(off + (size_t)(BH * n * d));
  w.vscale = off;
  off = align256(off + sizeof(float) * (size_t)(BH * d));
  w.vmax_partial = off;
  off = align256(off + sizeof(float) * (size_t)(BH * vq_chunks(n) * d));
  w.pack_partial2 = off;  // (last, so the regions above keep their offsets)
  off = align256(off + sizeof(double) * (size_t)(BH * pack_chunks(n) * d));
  w.total = off;
  return w;
}

}  // namespace had

using namespace had;

namespace {

bool debug_on() {
  static const bool on = [] {
    const char* e = getenv("HAD_DEBUG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

int fail(int status, const char* fn, const char* why) {
  if (debug_on()) fprintf(stderr, "[had] %s: %s (%s)\n", fn, had_status_str(status), why);
  return status;
}

// Total element count must stay addressable by the kernels' 32-bit row math.
bool sizes_ok(int64_t B, int64_t H, int64_t n, int64_t d) {
  if (B <= 0 || H <= 0 || n <= 0 || d <= 0) return false;
  const double total = (double)B * (double)H * (double)n * (double)d;
  return total < 2147483648.0;
}

int launch_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return HAD_OK;
  if (debug_on()) fprintf(stderr, "[had] %s: %s\n", fn, hipGetErrorString(e));
  return HAD_ERR_HIP;
}

int check_workspace(const void* ws, size_t bytes, int64_t B, int64_t H, int64_t n, int64_t d, const char* fn) {
  if (ws == nullptr) return fail(HAD_ERR_WORKSPACE, fn, "workspace is NULL");
  if (bytes < workspace_layout(B, H, n, d).total) return fail(HAD_ERR_WORKSPACE, fn, "workspace too small");
  if (((uintptr_t)ws & 255u) != 0) return fail(HAD_ERR_WORKSPACE, fn, "workspace not 256-byte aligned");
  return HAD_OK;
}

// Checks shared by the two attention entry points.
int check_attention(const uint32_t* qbits, const uint32_t* kbits, const void* v, int v_dtype, int64_t B,
                    int64_t H, int64_t n, int64_t d, float* out, const char* fn) {
  if (qbits == nullptr || kbits == nullptr || v == nullptr || out == nullptr)
    return fail(HAD_ERR_INVALID_ARG, fn, "NULL tensor");
  if (!sizes_ok(B, H, n, d)) return fail(HAD_ERR_INVALID_ARG, fn, "sizes must be positive and B*H*n*d < 2^31");
  if (v_dtype != HAD_F32 && v_dtype != HAD_BF16) return fail(HAD_ERR_INVALID_ARG, fn, "unknown v_dtype");
  if (d != 64 && d != 128) return fail(HAD_ERR_UNSUPPORTED, fn, "attention kernels take d = 64 or 128");
  if (n > HAD_MAX_N) return fail(HAD_ERR_UNSUPPORTED, fn, "n above HAD_MAX_N");
  return HAD_OK;
}

// Two-dimensional decomposable bias of the *_2d entry points (row == NULL: none).
struct Bias2dArgs {
  const float* row = nullptr;
  const float* col = nullptr;
  const float* cls = nullptr;
  int64_t gh = 0, gw = 0;
};

int check_bias2d(const Bias2dArgs& b, int64_t n, const char* fn) {
  if (b.row == nullptr) return HAD_OK;
  if (b.gh < 1 || b.gw < 1) return fail(HAD_ERR_INVALID_ARG, fn, "grid sizes must be positive");
  if (b.gh > 13000 || b.gw > 13000) return fail(HAD_ERR_UNSUPPORTED, fn, "grid too large for the position codes");
  if (n != b.gh * b.gw + (b.cls != nullptr ? 1 : 0))
    return fail(HAD_ERR_INVALID_ARG, fn, "n must be grid_h * grid_w, plus one with a class token");
  return HAD_OK;
}

void set_bias2d(AttnParams* p, const Bias2dArgs& b) {
  p->brow = b.row;
  p->bcol = b.col;
  p->bcls = b.cls;
  p->gh = (int)b.gh;
  p->gw = (int)b.gw;
  p->cls = b.cls != nullptr ? 1 : 0;
}

int64_t topn_max_n(int v_kind, int64_t d) { return topn_resident_max_n(v_kind, d); }

}  // namespace

namespace had {
// Largest n the resident top-N kernels handle (V of one head staged in LDS; at
// head_dim 128 the rows are twice as long).
int64_t topn_resident_max_n(int v_kind, int64_t d) {
  const int64_t base = v_kind == 0 ? 512 : 1024;
  return d == 128 ? base / 2 : base;
}
}  // namespace had

extern "C" {

int had_abi_version(void) { return HAD_ABI_VERSION; }

const char* had_status_str(int status) {
  switch (status) {
    case HAD_OK: return "HAD_OK";
    case HAD_ERR_INVALID_ARG: return "HAD_ERR_INVALID_ARG";
    case HAD_ERR_UNSUPPORTED: return "HAD_ERR_UNSUPPORTED";
    case HAD_ERR_WORKSPACE: return "HAD_ERR_WORKSPACE";
    case HAD_ERR_HIP: return "HAD_ERR_HIP";
    default: return "HAD_ERR_UNKNOWN";
  }
}

size_t had_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d) {
  if (!sizes_ok(B, H, n, d)) return 0;
  return workspace_layout(B, H, n, d).total;
}

int had_workspace_region(int64_t B, int64_t H, int64_t n, int64_t d, int region, size_t* offset, size_t* bytes) {
  if (offset == nullptr || bytes == nullptr || !sizes_ok(B, H, n, d)) return HAD_ERR_INVALID_ARG;
  const WorkspaceLayout w = workspace_layout(B, H, n, d);
  switch (region) {
    case HAD_WS_VQ:
      *offset = w.vq;
      *bytes = (size_t)(B * H * n * d);
      return HAD_OK;
    case HAD_WS_VSCALE:
      *offset = w.vscale;
      *bytes = sizeof(float) * (size_t)(B * H * d);
      return HAD_OK;
    default:
      return HAD_ERR_INVALID_ARG;
  }
}

namespace {

// Shared checks of had_pack and had_pack_qk; fills everything but the tensor sets.
int pack_common(int64_t B, int64_t H, int64_t n, int64_t d, int x_dtype, int mode, PackParams* p,
                const char* fn) {
  if (!sizes_ok(B, H, n, d)) return fail(HAD_ERR_INVALID_ARG, fn, "sizes must be positive and B*H*n*d < 2^31");
  if (x_dtype != HAD_F32 && x_dtype != HAD_BF16) return fail(HAD_ERR_INVALID_ARG, fn, "unknown x_dtype");
  if (mode != HAD_SIGN && mode != HAD_MEAN_SIGN) return fail(HAD_ERR_INVALID_ARG, fn, "unknown mode");
  if (d != 32 && d != 64 && d != 128) return fail(HAD_ERR_UNSUPPORTED, fn, "d must be 32, 64 or 128");
  if (n > HAD_MAX_N) return fail(HAD_ERR_UNSUPPORTED, fn, "n above HAD_MAX_N");
  p->x_dtype = x_dtype;
  p->BH = B * H;
  p->n = n;
  p->d = d;
  p->mode = mode;
  return HAD_OK;
}

}  // namespace

int had_pack(const void* x, int x_dtype, int64_t B, int64_t H, int64_t n, int64_t d, int mode, uint32_t* bits,
             float* alpha, float* mu, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "had_pack";
  if (x == nullptr || bits == nullptr) return fail(HAD_ERR_INVALID_ARG, fn, "NULL tensor");
  PackParams p{};
  int st = pack_common(B, H, n, d, x_dtype, mode, &p, fn);
  if (st != HAD_OK) return st;
  p.count = 1;
  p.set[0] = PackSet{x, bits, alpha, mu, nullptr};
  if (mode == HAD_MEAN_SIGN) {
    if (alpha == nullptr || mu == nullptr) return fail(HAD_ERR_INVALID_ARG, fn, "MEAN_SIGN needs alpha and mu");
    st = check_workspace(workspace, workspace_bytes, B, H, n, d, fn);
    if (st != HAD_OK) return st;
    p.set[0].partial =
        reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + workspace_layout(B, H, n, d).pack_partial);
  }
  return launch_status(launch_pack(p, static_cast<hipStream_t>(stream)), fn);
}

int had_pack_qk(const void* q, const void* k, int x_dtype, int64_t B, int64_t H, int64_t n, int64_t d, int mode,
                uint32_t* qbits, uint32_t* kbits, float* alpha_q, float* alpha_k, float* mu_q, float* mu_k,
                void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "had_pack_qk";
  if (q == nullptr || k == nullptr || qbits == nullptr || kbits == nullptr)
    return fail(HAD_ERR_INVALID_ARG, fn, "NULL tensor");
  PackParams p{};
  int st = pack_common(B, H, n, d, x_dtype, mode, &p, fn);
  if (st != HAD_OK) return st;
  p.count = 2;
  p.set[0] = PackSet{q, qbits, alpha_q, mu_q, nullptr};
  p.set[1] = PackSet{k, kbits, alpha_k, mu_k, nullptr};
  if (mode == HAD_MEAN_SIGN) {
    if (alpha_q == nullptr || alpha_k == nullptr || mu_q == nullptr || mu_k == nullptr)
      return fail(HAD_ERR_INVALID_ARG, fn, "MEAN_SIGN needs alpha and mu for Q and K");
    st = check_workspace(workspace, workspace_bytes, B, H, n, d, fn);
    if (st != HAD_OK) return st;
    const WorkspaceLayout w = workspace_layout(B, H, n, d);
    p.set[0].partial = reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + w.pack_partial);
    p.set[1].partial = reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + w.pack_partial2);
  }
  return launch_status(launch_pack(p, static_cast<hipStream_t>(stream)), fn);
}

static int topn_impl(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                     const float* bias_table, const Bias2dArgs& b2, const void* v, int v_dtype, int64_t B, int64_t H,
                     int64_t n, int64_t d, int64_t top_n, int av_mode, float* out, int32_t* idx_out, void* workspace,
                     size_t workspace_bytes, void* stream, const char* fn) {
  int st = check_attention(qbits, kbits, v, v_dtype, B, H, n, d, out, fn);
  if (st != HAD_OK) return st;
  st = check_bias2d(b2, n, fn);
  if (st != HAD_OK) return st;
  if (top_n < 1) return fail(HAD_ERR_INVALID_ARG, fn, "top_n must be >= 1");
  if (av_mode != HAD_AV_F32 && av_mode != HAD_AV_Q8 && av_mode != HAD_AV_Q4)
    return fail(HAD_ERR_INVALID_ARG, fn, "unknown av_mode");
  const int64_t keep = top_n < n ? top_n : n;
  const bool quant = av_mode != HAD_AV_F32;
  // V kinds: 0 f32, 1 bf16, 2 int8 codes, 3 4-bit codes two per byte
  const int v_kind = quant ? (av_mode == HAD_AV_Q4 ? 3 : 2) : (v_dtype == HAD_BF16 ? 1 : 0);
  // above the resident limit: the streaming kernel while its candidate buffer holds
  // the kept set, the threshold-first kernel beyond
  const bool streaming = n > topn_max_n(v_kind, d);
  const int64_t tab = b2.row != nullptr ? bias2d_floats(b2.gh, b2.gw, b2.cls != nullptr) : 0;
  const bool wide = streaming && !topn_stream_takes(n, keep, tab);
  if (wide && tab > topn_wide_bias2d_max())
    return fail(HAD_ERR_UNSUPPORTED, fn, "grid too long for the long-sequence kernels' bias tables");
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnParams p{};
  p.qbits = qbits;
  p.kbits = kbits;
  p.alpha_q = alpha_q;
  p.alpha_k = alpha_k;
  p.bias = bias_table;
  set_bias2d(&p, b2);
  p.v = v;
  p.v_kind = v_kind;
  p.B = B;
  p.H = H;
  p.n = n;
  p.d = d;
  p.keep = keep;
  p.out = out;
  p.idx = idx_out;
  if (quant) {
    st = check_workspace(workspace, workspace_bytes, B, H, n, d, fn);
    if (st != HAD_OK) return st;
    const WorkspaceLayout w = workspace_layout(B, H, n, d);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    VQuantParams q{};
    q.v = v;
    q.v_dtype = v_dtype;
    q.BH = B * H;
    q.n = n;
    q.d = d;
    q.vmax_partial = reinterpret_cast<float*>(ws + w.vmax_partial);
    q.vscale = reinterpret_cast<float*>(ws + w.vscale);
    q.vq = reinterpret_cast<int8_t*>(ws + w.vq);
    q.levels = av_mode == HAD_AV_Q4 ? 7 : 127;
    hipError_t e = launch_vquant(q, s);
    if (e != hipSuccess) return launch_status(e, fn);
    p.v = q.vq;
    p.vscale = q.vscale;
  }
  // the matrix-core kernel first: at head_dim 128 it holds up to 1024 keys, past the
  // resident kernel's limit
  if (topn_mfma_supported(p)) return launch_status(launch_topn_mfma(p, s), fn);
  if (wide) return launch_status(launch_topn_wide(p, s), fn);
  if (streaming) return launch_status(launch_topn_stream(p, s), fn);
  return launch_status(launch_topn(p, s), fn);
}

int had_attention_topn(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                       const float* bias_table, const void* v, int v_dtype, int64_t B, int64_t H, int64_t n,
                       int64_t d, int64_t top_n, int av_mode, float* out, int32_t* idx_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return topn_impl(qbits, kbits, alpha_q, alpha_k, bias_table, Bias2dArgs{}, v, v_dtype, B, H, n, d, top_n, av_mode,
                   out, idx_out, workspace, workspace_bytes, stream, "had_attention_topn");
}

int had_attention_topn_2d(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                          const float* row_table, const float* col_table, const float* cls_table, int64_t grid_h,
                          int64_t grid_w, const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                          int64_t top_n, int av_mode, float* out, int32_t* idx_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  static const char* fn = "had_attention_topn_2d";
  if (row_table == nullptr || col_table == nullptr) return fail(HAD_ERR_INVALID_ARG, fn, "NULL bias table");
  return topn_impl(qbits, kbits, alpha_q, alpha_k, nullptr, Bias2dArgs{row_table, col_table, cls_table, grid_h, grid_w},
                   v, v_dtype, B, H, n, d, top_n, av_mode, out, idx_out, workspace, workspace_bytes, stream, fn);
}

// Every check of the dense entry points except the workspace's.
static int dense_checks(const uint32_t* qbits, const uint32_t* kbits, const Bias2dArgs& b2, const void* v, int v_dtype,
                        int64_t B, int64_t H, int64_t n, int64_t d, float* out, const char* fn) {
  int st = check_attention(qbits, kbits, v, v_dtype, B, H, n, d, out, fn);
  if (st != HAD_OK) return st;
  st = check_bias2d(b2, n, fn);
  if (st != HAD_OK) return st;
  if (n > dense_q8_max_n() && b2.row != nullptr &&
      bias2d_floats(b2.gh, b2.gw, b2.cls != nullptr) > dense_long_bias2d_max())
    return fail(HAD_ERR_UNSUPPORTED, fn, "grid too long for the long-sequence dense kernel's bias tables");
  return HAD_OK;
}

static int dense_impl(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                      const float* bias_table, const Bias2dArgs& b2, const void* v, int v_dtype, int64_t B, int64_t H,
                      int64_t n, int64_t d, float* out, void* workspace, size_t workspace_bytes, void* stream,
                      const char* fn) {
  int st = dense_checks(qbits, kbits, b2, v, v_dtype, B, H, n, d, out, fn);
  if (st != HAD_OK) return st;
  st = check_workspace(workspace, workspace_bytes, B, H, n, d, fn);
  if (st != HAD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const WorkspaceLayout w = workspace_layout(B, H, n, d);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  VQuantParams q{};
  q.v = v;
  q.v_dtype = v_dtype;
  q.BH = B * H;
  q.n = n;
  q.d = d;
  q.vmax_partial = reinterpret_cast<float*>(ws + w.vmax_partial);
  q.vscale = reinterpret_cast<float*>(ws + w.vscale);
  q.vq = reinterpret_cast<int8_t*>(ws + w.vq);
  q.levels = 127;
  hipError_t e = launch_vquant(q, s);
  if (e != hipSuccess) return launch_status(e, fn);
  AttnParams p{};
  p.qbits = qbits;
  p.kbits = kbits;
  p.alpha_q = alpha_q;
  p.alpha_k = alpha_k;
  p.bias = bias_table;
  set_bias2d(&p, b2);
  p.v = q.vq;
  p.v_kind = 2;
  p.vscale = q.vscale;
  p.B = B;
  p.H = H;
  p.n = n;
  p.d = d;
  p.keep = n;
  p.out = out;
  p.idx = nullptr;
  if (n > dense_q8_max_n()) return launch_status(launch_dense_long(p, s), fn);
  return launch_status(launch_dense_q8(p, s), fn);
}

int binattn_dense_q8(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                     const float* bias_table, const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                     float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return had::dense_q8_entry(qbits, kbits, alpha_q, alpha_k, bias_table, v, v_dtype, B, H, n, d, out, workspace,
                             workspace_bytes, stream, "binattn_dense_q8");
}

}  // extern "C"

namespace had {
int dense_q8_entry(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                   const float* bias_table, const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                   float* out, void* workspace, size_t workspace_bytes, void* stream, const char* fn) {
  return dense_impl(qbits, kbits, alpha_q, alpha_k, bias_table, Bias2dArgs{}, v, v_dtype, B, H, n, d, out, workspace,
                    workspace_bytes, stream, fn);
}

int dense_q8_check(const uint32_t* qbits, const uint32_t* kbits, const void* v, int v_dtype, int64_t B, int64_t H,
                   int64_t n, int64_t d, float* out, const char* fn) {
  return dense_checks(qbits, kbits, Bias2dArgs{}, v, v_dtype, B, H, n, d, out, fn);
}

int report(int status, const char* fn, const char* why) { return fail(status, fn, why); }
}  // namespace had

extern "C" {

int binattn_dense_q8_2d(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q, const float* alpha_k,
                        const float* row_table, const float* col_table, const float* cls_table, int64_t grid_h,
                        int64_t grid_w, const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d,
                        float* out, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "binattn_dense_q8_2d";
  if (row_table == nullptr || col_table == nullptr) return fail(HAD_ERR_INVALID_ARG, fn, "NULL bias table");
  return dense_impl(qbits, kbits, alpha_q, alpha_k, nullptr, Bias2dArgs{row_table, col_table, cls_table, grid_h, grid_w},
                    v, v_dtype, B, H, n, d, out, workspace, workspace_bytes, stream, fn);
}

int had_attention_topn_fused(const void* q, const void* k, int qk_dtype, int mode, const float* bias_table,
                             const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d, int64_t top_n,
                             float* out, int32_t* idx_out, void* stream) {
  static const char* fn = "had_attention_topn_fused";
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return fail(HAD_ERR_INVALID_ARG, fn, "NULL tensor");
  if (!sizes_ok(B, H, n, d)) return fail(HAD_ERR_INVALID_ARG, fn, "sizes must be positive and B*H*n*d < 2^31");
  if (qk_dtype != HAD_F32 && qk_dtype != HAD_BF16) return fail(HAD_ERR_INVALID_ARG, fn, "unknown qk_dtype");
  if (v_dtype != HAD_F32 && v_dtype != HAD_BF16) return fail(HAD_ERR_INVALID_ARG, fn, "unknown v_dtype");
  if (mode != HAD_SIGN && mode != HAD_MEAN_SIGN) return fail(HAD_ERR_INVALID_ARG, fn, "unknown mode");
  if (top_n < 1) return fail(HAD_ERR_INVALID_ARG, fn, "top_n must be >= 1");
  if (d != 64 && d != 128) return fail(HAD_ERR_UNSUPPORTED, fn, "d must be 64 or 128");
  const int v_kind = v_dtype == HAD_BF16 ? 1 : 0;
  if (n > topn_max_n(v_kind, d)) return fail(HAD_ERR_UNSUPPORTED, fn, "n above what one workgroup holds on chip");
  if (mode == HAD_MEAN_SIGN && n > 256) return fail(HAD_ERR_UNSUPPORTED, fn, "mean-centred codes: n above 256");
  AttnParams p{};
  p.xq = q;
  p.xk = k;
  p.qk_bf16 = qk_dtype == HAD_BF16;
  p.mean = mode == HAD_MEAN_SIGN;
  p.bias = bias_table;
  p.v = v;
  p.v_kind = v_kind;
  p.B = B;
  p.H = H;
  p.n = n;
  p.d = d;
  p.keep = top_n < n ? top_n : n;
  p.out = out;
  p.idx = idx_out;
  return launch_status(launch_topn(p, static_cast<hipStream_t>(stream)), fn);
}

int binattn_dense_q8_fused(const void* q, const void* k, int qk_dtype, int mode, const float* bias_table,
                           const void* v, int v_dtype, int64_t B, int64_t H, int64_t n, int64_t d, float* out,
                           void* stream) {
  static const char* fn = "binattn_dense_q8_fused";
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return fail(HAD_ERR_INVALID_ARG, fn, "NULL tensor");
  if (!sizes_ok(B, H, n, d)) return fail(HAD_ERR_INVALID_ARG, fn, "sizes must be positive and B*H*n*d < 2^31");
  if (qk_dtype != HAD_F32 && qk_dtype != HAD_BF16) return fail(HAD_ERR_INVALID_ARG, fn, "unknown qk_dtype");
  if (v_dtype != HAD_F32 && v_dtype != HAD_BF16) return fail(HAD_ERR_INVALID_ARG, fn, "unknown v_dtype");
  if (mode != HAD_SIGN && mode != HAD_MEAN_SIGN) return fail(HAD_ERR_INVALID_ARG, fn, "unknown mode");
  if (d != 64 && d != 128) return fail(HAD_ERR_UNSUPPORTED, fn, "d must be 64 or 128");
  if (n > dense_q8_max_n()) return fail(HAD_ERR_UNSUPPORTED, fn, "n above what one workgroup stages");
  DenseFusedParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.qk_dtype = qk_dtype;
  p.v_dtype = v_dtype;
  p.mode = mode;
  p.bias = bias_table;
  p.B = B;
  p.H = H;
  p.n = n;
  p.d = d;
  p.out = out;
  return launch_status(launch_dense_q8_fused(p, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
