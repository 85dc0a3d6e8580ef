// moe_forward_noalloc: the layer forward with its workspace in a fixed,
// library-owned device array, for callers that cannot allocate (graph
// capture, serving loops).  The array is a file-scope __device__ variable:
// each GPU the library runs on holds its own copy from the moment the code
// object is loaded there until the process ends.  Host code never passes
// the array's name to a kernel (in host code it names a host-side stand-in);
// it looks up the device address once per device with hipGetSymbolAddress
// and uses that pointer.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/moe_mi355x.h"
#include "api_internal.h"

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).
moe_status_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[160];
    std::snprintf(msg, sizeof msg, "moe_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return moe::set_error(MOE_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return moe::set_error(MOE_ERR_INVALID_ARGUMENT, "moe_forward_noalloc: device id above 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      std::snprintf(msg, sizeof msg, "moe_forward_noalloc: hipGetSymbolAddress(scratch): %s",
                    hipGetErrorString(e));
      return moe::set_error(MOE_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_forward_noalloc(const moe_problem_t* p, const moe_weights_t* w,
                                            const uint16_t* x, const float* beta_in,
                                            uint16_t* y, moe_aux_t* aux, void* stream) {
  const size_t need = moe_forward_workspace_bytes(p);
  if (need == 0)  // an invalid problem: the checks of the forward report why
    return moe::forward_bf16(p, w, x, beta_in, y, aux, nullptr, 0, stream, true);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "moe_forward_noalloc: the problem needs %zu bytes of workspace, above the "
                  "fixed %zu of the no-allocation path (use moe_forward)",
                  need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    return moe::set_error(MOE_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  void* ws = nullptr;
  const moe_status_t s = scratch_on_current_device(&ws);
  if (s != MOE_OK) return s;
  return moe::forward_bf16(p, w, x, beta_in, y, aux, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                           stream, true);
}
