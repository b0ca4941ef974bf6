// kdn_noalloc.hip -- the device scratch of kdn_backward_noalloc: the backward's
// workspace for callers that cannot allocate device memory.
//
// The scratch is a file-scope device array of kNoallocScratchBytes.  Each
// device the library runs on holds its own copy until the process ends.  In
// host code the array's name is only a stand-in, never a device address: the
// address of the current device's copy comes from hipGetSymbolAddress, once
// per device (with that device current), and is cached here.
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace kdn {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace kdn
