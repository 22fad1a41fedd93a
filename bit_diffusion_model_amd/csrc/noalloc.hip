// The forward without any allocation: svdq_linear_forward's two kernels with their
// workspace in a fixed device array of this library, for callers that cannot allocate
// device memory (code under stream capture into a HIP graph, serving loops that must not
// allocate).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/svdq.h"
#include "internal.hpp"

namespace svdq {
namespace {

// The workspace of every call on a device: one copy per device, alive until the process
// ends.  In host code `scratch` names a host-side stand-in; kernels receive the device
// address obtained below.
static __device__ __align__(256) uint8_t scratch[SVDQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up once per device with
// that device current (the caller's current device).
svdq_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SVDQ_EUNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(SVDQ_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SVDQ_OK;
}

}  // namespace
}  // namespace svdq

extern "C" svdq_status svdq_linear_forward_noalloc(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx,
                                                   void* Y, int64_t ldy, int32_t ydtype, void* stream) {
  using namespace svdq;
  if (!layer) return fail(SVDQ_EINVAL, "layer is NULL");
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  const size_t need = svdq_workspace_bytes(layer, M);
  if (need == 0) return fail(SVDQ_EINVAL, "bad layer dimensions or format");
  if (need > (size_t)SVDQ_NOALLOC_SCRATCH_BYTES)
    return fail(SVDQ_EUNSUPPORTED, "this layer at M = %lld needs %zu bytes of workspace, more than the %zu of the "
                "fixed scratch array: call svdq_linear_forward with a workspace instead", (long long)M, need,
                (size_t)SVDQ_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  svdq_status st = scratch_ptr(&ws);
  if (st != SVDQ_OK) return st;
  return linear_forward(layer, M, X, ldx, Y, ldy, ydtype, ws, (size_t)SVDQ_NOALLOC_SCRATCH_BYTES, stream);
}
