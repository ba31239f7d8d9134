// Library-owned device scratch for the allocation-free entry point.
//
// Some callers cannot allocate device memory for a call (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).  For
// them the conv2d backward can take its fp64 partial sums from this
// file-scope array instead of a caller-given workspace.  Each GPU the library
// runs on holds its own copy of the array, at its own address, until the
// process ends.
//
// In host code the array's name is only a host-side stand-in, never a
// device address.  The device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept; host code uses
// that address, never the name.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "scratch.h"

namespace dw {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace dw
