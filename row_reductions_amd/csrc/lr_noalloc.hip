// The device array behind lr_run_f32_noalloc (lr_abi.cpp), the entry point
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  The
// split-row partials that lr_run_f32 keeps in a caller workspace go to this
// library-owned array instead, `scratch`, of LR_NOALLOC_SCRATCH_BYTES bytes;
// every GPU the library runs on holds its own copy of it until the process
// ends.
//
// In host code `scratch` names a host-side stand-in, not a device address:
// its address on each device is looked up once per device (with that device
// current) through hipGetSymbolAddress and kept in `g_scratch`; only that
// pointer is ever passed to a kernel.  Nothing here allocates or frees
// memory.  Every call on one GPU shares that GPU's array: the split kernels
// write every partial before they read it, so nothing has to be cleared
// between calls, but calls that overlap in time on one GPU (other streams,
// other host threads) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lr_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[LR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device.
lr_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LR_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LR_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LR_OK;
}

}  // namespace

namespace lr {

lr_status noalloc_scratch(void** out) { return scratch_of_current_device(out); }

}  // namespace lr
