// ffd_scratch.hip -- the library's own fixed scratch area, for the decode entry point that
// allocates nothing (ffd_decode_sparse_noalloc).
//
// The area is a file-scope device array.  In host code its name is only a host-side stand-in for
// the symbol, not a device address, so the address every kernel argument and launch uses is
// looked up with hipGetSymbolAddress: once per device, with that device current, at the first
// call on it.  Each GPU holds its own copy of the array (at its own address) until the process
// ends.  That first call also zeroes the area's counter region with a kernel on the caller's
// stream; every completed decode returns the counters it used to zero, so later calls find them
// cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ffd_internal.h"

namespace ffd {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // the device address of `scratch` on each device, once looked up

}  // namespace

hipError_t scratch_area(size_t counter_bytes, hipStream_t stream, void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        e = launch_zero_counters(static_cast<uint32_t*>(p), (int)(counter_bytes / sizeof(uint32_t)),
                                 stream);
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace ffd
