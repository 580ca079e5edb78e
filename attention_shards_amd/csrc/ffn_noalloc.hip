// tp_ffn_shard_noalloc: the FFN shard (column-parallel W1 + GeLU, then
// row-parallel W2) for callers that cannot allocate device memory.  The
// kernels and their sequence are tp_ffn_shard's; the only difference is
// where GeLU(Z_i) lives between the two products: a file-scope device array
// (`scratch`) instead of a caller-provided workspace.
//
// The array's name is a host-side stand-in in host code, not a device
// address, so its address on the current device is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// pointer is passed on.  Each GPU holds its own copy at its own address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/tp_shard.h"
#include "internal.h"

namespace {

__device__ __align__(256) uint8_t scratch[TP_FFN_NOALLOC_MAX_WORKSPACE];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The current device's copy of the array (looked up on first use).
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" tp_status_t tp_ffn_shard_noalloc(const void* X, const void* W1_i, const void* W2_i,
                                            void* Y_i, int64_t tokens, int64_t hidden,
                                            int64_t ffn, int32_t i, int32_t t, int64_t ld_w1,
                                            int32_t in_dtype, int32_t out_dtype, void* stream) {
  const char* fn = "tp_ffn_shard_noalloc";
  try {
    tp_status_t st = tp::ffn_check_args(fn, X, W1_i, W2_i, Y_i, tokens, hidden, ffn, i, t,
                                        ld_w1, in_dtype, out_dtype);
    if (st != TP_SUCCESS) return st;
    if (tokens == 0) return TP_SUCCESS;
    const size_t need = tp_ffn_shard_workspace_bytes(tokens, hidden, ffn, t, in_dtype);
    if (need > TP_FFN_NOALLOC_MAX_WORKSPACE) {
      char msg[256];
      snprintf(msg, sizeof(msg),
               "%s(i=%d): GeLU(Z_i) needs %zu bytes, above the %zu-byte scratch array "
               "(use tp_ffn_shard with a workspace)",
               fn, i, need, (size_t)TP_FFN_NOALLOC_MAX_WORKSPACE);
      return tp::set_error(TP_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) {
      char msg[256];
      snprintf(msg, sizeof(msg), "%s: device address of the scratch array: %s", fn,
               hipGetErrorString(e));
      return tp::set_error(TP_ERR_HIP, msg);
    }
    return tp_ffn_shard(X, W1_i, W2_i, Y_i, tokens, hidden, ffn, i, t, ld_w1, in_dtype,
                        out_dtype, ws, TP_FFN_NOALLOC_MAX_WORKSPACE, stream);
  } catch (...) {
    return tp::set_error(TP_ERR_HIP, "tp_ffn_shard_noalloc: internal exception");
  }
}
