// The library-owned scratch buffer of flash_deform_attn_backward_noalloc:
// a file-scope device array, one copy per device, used in place of the
// caller's workspace by callers that cannot allocate device memory.
//
// The array's name is a host-side stand-in in host code, not a device
// address, so host code never uses it directly: the first call on a device
// (with that device current) looks up the device address with
// hipGetSymbolAddress and keeps it per device; every launch receives that
// address as its workspace argument.

#include "dcnv4_internal.h"
#include "fdattn_internal.h"

#include <mutex>

namespace fdattn {
namespace {

constexpr int kMaxDevices = 64;

// Zero-initialised device memory (no file space: it is not initialised
// data); held by every device the library runs on until the process ends.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];   // device address of scratch, per device (null: not looked up yet)

}  // namespace

hipError_t noalloc_scratch(void **ptr)
{
    *ptr = nullptr;
    int dev = 0;
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

}  // namespace fdattn
