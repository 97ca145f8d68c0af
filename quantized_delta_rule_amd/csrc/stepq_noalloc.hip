// stepq_noalloc.hip -- the device scratch of the no-allocation decode entry point.
//
// A split-mode step hands the readout kernel's per-tile update factors (a_i, beta k_i and the
// per-column error or u, v) to the side-stream writeback kernel through a buffer.  The regular
// entry point uses a buffer the plan allocated; stepq_decode_step_noalloc uses this file-scope
// array instead, so the call itself allocates nothing.  Each GPU the library runs on holds its
// own copy of the array until the process ends.
//
// The array's name is a host-side stand-in in host code, not a device address: host code uses
// only the address hipGetSymbolAddress returns for the current device, resolved once per device
// by scratch_resolve (called at plan creation, with the plan's device current).
#include <hip/hip_runtime.h>

#include <mutex>

#include "stepq_internal.h"

namespace stepq {

// hand-over of up to kScratchBytes / (16 d) tiles: [B * n_heads][4 d] floats
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this device's scratch array (the current device must be `device`).
// Resolves it on first use per device.  Returns 0 or a negative STEPQ_ERR_* code via fail().
int scratch_resolve(int device, void** out) {
  if (device < 0 || device >= kMaxDevices)
    return fail(-2 /* STEPQ_ERR_UNSUPPORTED */, "device %d beyond the %d devices the scratch "
                "table covers", device, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(-3 /* STEPQ_ERR_HIP */, "hipGetSymbolAddress(scratch) on device %d: %s",
                  device, hipGetErrorString(e));
    g_ptr[device] = p;
  }
  *out = g_ptr[device];
  return 0;
}

}  // namespace stepq
