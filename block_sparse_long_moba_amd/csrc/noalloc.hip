// The forward pass without allocation, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): moba_fwd_ex on a workspace the library owns, a static device
// array of MOBA_NOALLOC_WORKSPACE_BYTES. Each GPU the library runs on holds
// its own copy of the array until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is ever handed to kernels.
#include <stdio.h>

#include <mutex>

#include "moba_internal.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[MOBA_NOALLOC_WORKSPACE_BYTES];

std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device

// Device address of the current device's copy of `scratch` (looked up on the
// first call on that device). Returns the HIP error of the lookup.
hipError_t scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" moba_status_t moba_fwd_noalloc(const void *q, const void *k, const void *v,
                                          const int32_t *cu_seqlens, const moba_shape_t *shape,
                                          int32_t block_size, int32_t topk, float softmax_scale,
                                          void *out, float *lse, hipStream_t stream) {
  const size_t cap = (size_t)MOBA_NOALLOC_WORKSPACE_BYTES;
  // the smallest plan (one kv head per pass) must fit the static workspace;
  // moba_fwd_ex then takes the largest pass that fits it. Invalid arguments
  // (size 0) are left to moba_fwd_ex, which names the problem.
  const size_t need = moba_fwd_workspace_size(shape, block_size, topk, 1);
  if (need > cap) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "moba_fwd_noalloc: this shape needs %zu bytes of workspace (one kv head per pass); "
             "the static workspace holds %zu",
             need, cap);
    return moba::report_error(MOBA_ERROR_UNSUPPORTED, msg);
  }
  void *ws = nullptr;
  if (need > 0 && shape->total_tokens > 0) {
    const hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess) {
      char msg[256];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress: %s", hipGetErrorString(e));
      return moba::report_error(MOBA_ERROR_HIP, msg);
    }
  }
  return moba_fwd_ex(q, k, v, cu_seqlens, shape, block_size, topk, softmax_scale, out, lse, ws,
                     cap, stream);
}
