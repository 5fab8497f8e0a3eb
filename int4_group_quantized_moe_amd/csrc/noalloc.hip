// moe_layer_forward without a caller-provided workspace, for callers that
// cannot allocate device memory: code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc.  The workspace is a fixed-size
// device array of this library, one per GPU, held until the process ends.
#include <mutex>

#include "host.h"
#include "moe_internal.h"

namespace moe {
namespace {

// The library's scratch.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is ever passed to the kernels.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device

// Device address of the current device's scratch (looked up on the first
// call on that device, with the device current).  MOE_OK or a status.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_NO_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_layer_forward_noalloc(const moe_layer_desc* desc, const void* x,
                                         const float* router_w, const float* router_bias,
                                         const void* expert_slab, const int32_t* slot_table,
                                         const void* shared_blob, void* out,
                                         hipStream_t stream) {
  MOE_TRY(check_shape(desc));
  if (desc->n_tokens == 0) return MOE_OK;
  if (make_ws_plan(*desc).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return MOE_ERR_NO_DEVICE;
  void* ws = nullptr;
  MOE_TRY(scratch_address(&ws));
  // every kernel of a layer call writes the workspace words it reads, so the
  // previous call's contents need no clearing
  return moe_layer_forward(desc, x, router_w, router_bias, expert_slab, slot_table, shared_blob,
                           out, ws, stream);
}
