// moe_grouped_ffn_noalloc: the grouped expert FFN with its workspace in a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation).  What it computes, and its limits, are documented in
// include/moe_layer.h.
#include <mutex>

#include "kernels.h"
#include "moe_layer.h"

namespace {

// The workspace: each GPU the library runs on holds its own copy from the
// time the library's code is loaded on it until the process ends.  In host
// code `scratch` is only a stand-in for the symbol: its device address on the
// current GPU comes from hipGetSymbolAddress (scratch_on_current_device).
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (guarded by g_mu)

// The address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
moe_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return (moe_status)moe::set_last_error(MOE_EHIP, "moe_grouped_ffn_noalloc: hipGetDevice: %s",
                                           hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return (moe_status)moe::set_last_error(MOE_EUNSUPPORTED,
                                           "moe_grouped_ffn_noalloc: device %d (at most %d devices)",
                                           dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return (moe_status)moe::set_last_error(
          MOE_EHIP, "moe_grouped_ffn_noalloc: hipGetSymbolAddress of the scratch array: %s",
          hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_grouped_ffn_noalloc(const void* x, moe_dtype dt, int64_t T, int H,
                                              int I, int E, int K, const void* w13, const void* w2,
                                              const moe_plan* plan, void* y_pairs, void* stream) {
  if (!plan) return (moe_status)moe::set_last_error(MOE_EINVAL, "moe_grouped_ffn_noalloc: plan is NULL");
  const int64_t need = moe_ffn_workspace_bytes(plan->cap, I);
  if (need < 0)
    return (moe_status)moe::set_last_error(MOE_EINVAL, "moe_grouped_ffn_noalloc: plan->cap = %lld, I = %d",
                                           (long long)plan->cap, I);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return (moe_status)moe::set_last_error(
        MOE_ECAPACITY,
        "moe_grouped_ffn_noalloc: this plan needs %lld bytes of workspace, more than the %lld of "
        "the allocation-free variant (use moe_grouped_ffn with a caller workspace)",
        (long long)need, (long long)MOE_NOALLOC_SCRATCH_BYTES);
  // an empty batch is checked and returns without touching the device
  void* ws = nullptr;
  if (T > 0) {
    moe_status st = scratch_on_current_device(&ws);
    if (st != MOE_OK) return st;
  }
  return moe_grouped_ffn(x, dt, T, H, I, E, K, w13, w2, plan, ws, MOE_NOALLOC_SCRATCH_BYTES, y_pairs,
                         stream);
}
