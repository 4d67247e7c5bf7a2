// noalloc_scratch.hip -- the library's own device scratch for
// moe_route_dispatch_noalloc: a fixed array in every GPU's memory, used in
// place of a caller-allocated workspace by callers that cannot allocate.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (with that device current)
// and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"
#include "moe_route.h"

namespace moe {
namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lookup;
std::atomic<void *> g_addr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = g_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (!p)
                return hipErrorInvalidSymbol;
            g_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace moe
