// contract_check.hip -- the per-device word that a build with contract checks
// (SA_CHECKED) sets bits in when its kernels meet a device table that breaks
// the caller's contract (sparse_attn_check_flags reads and clears it).  Other
// builds hold no such word.
//
// As with every file-scope device array, host code never passes the symbol
// itself to a kernel or a copy: its device address is looked up once per
// device (with that device current) and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sa_internal.hpp"

#ifdef SA_CHECKED
namespace {

static __device__ __align__(256) uint32_t contract_bits[64];   // word 0 is used; one line to itself

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint32_t *g_ptr[kMaxDevices];

} // namespace
#endif

namespace sa {

bool contract_checked()
{
#ifdef SA_CHECKED
    return true;
#else
    return false;
#endif
}

hipError_t contract_word(uint32_t **ptr)
{
    *ptr = nullptr;
#ifdef SA_CHECKED
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(contract_bits));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_ptr[dev] = static_cast<uint32_t *>(p);
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
#else
    return hipErrorNotSupported;
#endif
}

} // namespace sa
