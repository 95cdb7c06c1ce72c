// fwd_noalloc.hip -- device scratch for the attention call that allocates
// nothing (sparse_attn_fwd_noalloc): the split partials that sparse_attn_fwd
// keeps in a caller workspace live here in a fixed array of every GPU the
// library runs on, held until the process ends.
//
// Host code never passes `scratch` itself to a kernel or a copy: on the host
// that name is only a stand-in for the symbol.  The array's device address is
// looked up once per device (with that device current) and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sa_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[sa::kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];          // device address of `scratch` on each device, once looked up

} // namespace

namespace sa {

// Device address of the scratch array on the current device.  The first call on
// a device looks it up; later calls return the kept address.
hipError_t noalloc_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

} // namespace sa
