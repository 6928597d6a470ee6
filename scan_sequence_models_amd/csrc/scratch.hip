// scratch.hip -- the fixed device scratch of scan_fwd_noalloc: a file-scope
// array that each GPU the library runs on holds from the time the library's
// code is loaded there until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol);
// it asks the runtime once per device for the array's device address and
// hands kernels that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdscan.h"
#include "kernels.hpp"

static __device__ __align__(256) unsigned char scratch[SCAN_NOALLOC_MAX_WORKSPACE];

namespace gds {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gds
