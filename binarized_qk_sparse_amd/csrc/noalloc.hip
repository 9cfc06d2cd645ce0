// binattn_dense_q8_noalloc: the dense BinaryAttention forward (section 2.4,
// uint8 A times per-channel int8 V) with its scratch in a static device array
// instead of a caller-supplied workspace, for callers that cannot allocate.
//
// The array is a file-scope __device__ object.  Its name is only a host-side
// stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current (on the
// entry point's first call there), and only that address reaches the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/had.h"
#include "had_internal.h"

namespace had {
namespace {

constexpr size_t kScratchBytes = HAD_NOALLOC_SCRATCH_BYTES;
// Nothing in it needs clearing: every kernel of the dense path writes the
// integer V, the scales and the partial maxima before reading them.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array; hipGetSymbolAddress
// runs once per device.
int scratch_address(void** out, const char* fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return report(HAD_ERR_HIP, fn, "no current HIP device");
  if (dev >= kMaxDevices) return report(HAD_ERR_UNSUPPORTED, fn, "device index above the scratch table");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return report(HAD_ERR_HIP, fn, "hipGetSymbolAddress of the scratch failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HAD_OK;
}

}  // namespace
}  // namespace had

extern "C" int binattn_dense_q8_noalloc(const uint32_t* qbits, const uint32_t* kbits, const float* alpha_q,
                                        const float* alpha_k, const float* bias_table, const void* v, int v_dtype,
                                        int64_t B, int64_t H, int64_t n, int64_t d, float* out, void* stream) {
  static const char* fn = "binattn_dense_q8_noalloc";
  // every argument check first, so that an error status means no HIP call was made
  int st = had::dense_q8_check(qbits, kbits, v, v_dtype, B, H, n, d, out, fn);
  if (st != HAD_OK) return st;
  if (had_workspace_bytes(B, H, n, d) > had::kScratchBytes)
    return had::report(HAD_ERR_UNSUPPORTED, fn, "sizes need more than the static scratch");
  void* ws = nullptr;
  st = had::scratch_address(&ws, fn);
  if (st != HAD_OK) return st;
  return had::dense_q8_entry(qbits, kbits, alpha_q, alpha_k, bias_table, v, v_dtype, B, H, n, d, out, ws,
                             had::kScratchBytes, stream, fn);
}
