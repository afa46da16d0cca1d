// noalloc.hip -- the static device scratch behind ssd_forward_noalloc, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope __device__ array.  In host code its name is only
// a host-side stand-in, never a device address: the device address is taken
// here, once per device with that device current, with hipGetSymbolAddress,
// and cached per device.  Every kernel that uses the scratch receives that
// cached pointer.  Each GPU the library runs on holds its own copy of the array
// until the process ends; all calls on one GPU share it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace ssd {

namespace {

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || reinterpret_cast<uintptr_t>(p) % 256) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace ssd
