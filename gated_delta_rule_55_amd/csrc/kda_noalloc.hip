// kda_noalloc.hip -- the device scratch of kda_chunk_fwd_noalloc: a file-scope
// static device array that stands in for the caller's workspace, so that the
// entry point allocates nothing (for callers under graph capture or in loops
// that cannot call hipMalloc).
//
// Each GPU the library runs on holds its own copy of the array, from the first
// call on that device until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in, not a device
// address): its device address is looked up once per device with
// hipGetSymbolAddress and kept, and that address is what the kernels receive.
#include <mutex>

#include "kda_internal.h"

namespace kda {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
