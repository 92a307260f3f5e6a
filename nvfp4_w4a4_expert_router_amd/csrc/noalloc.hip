// moe_layer_forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the workspace is a file-scope device array of fixed size instead of a
// caller buffer.  Each GPU the library runs on holds its own copy of the array
// until the process ends; its device address is looked up once per device (on
// the first call with that device current) and kept.  Nothing in the
// workspace needs to start at zero: every kernel of the layer writes its
// scratch before reading it, so the previous call's contents are harmless.
// Calls that overlap in time on one GPU (two streams, two threads) share the
// array and race.
#include <mutex>

#include "common.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch` (its device address, never the
// host-side name of the array)
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_layer_forward_noalloc(const moe_layer* L, const uint16_t* x, int64_t T, const uint16_t* residual,
                              int32_t* topk_idx, float* topk_w, int32_t* expert_off, int32_t* row2pair,
                              int32_t* pair2row, float* y_rows, float* y_shared, uint16_t* out,
                              const moe_debug* dbg, hipStream_t stream) {
  if (!L) return MOE_EINVAL;
  if (T == 0) return moe_layer_forward(L, x, T, residual, topk_idx, topk_w, expert_off, row2pair, pair2row, y_rows,
                                       y_shared, out, dbg, nullptr, 0, stream);
  const size_t need = moe_workspace_bytes(L, T);
  if (need == 0)  // invalid layer or token count: the regular entry point names the error
    return moe_layer_forward(L, x, T, residual, topk_idx, topk_w, expert_off, row2pair, pair2row, y_rows, y_shared,
                             out, dbg, nullptr, 0, stream);
  if (need > kScratchBytes) return MOE_EWORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  return moe_layer_forward(L, x, T, residual, topk_idx, topk_w, expert_off, row2pair, pair2row, y_rows, y_shared, out,
                           dbg, ws, kScratchBytes, stream);
}

}  // extern "C"
