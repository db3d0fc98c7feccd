// moe_noalloc.hip -- the fixed device buffer behind moe_layer_decode_noalloc,
// for callers that cannot allocate (code under hipGraph capture, serving loops
// that forbid allocation).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy from module load until the process ends.  In host code its name
// is only a stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and that address is what the
// kernels receive.  Calls on one GPU share its array and must not overlap.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[moe::kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];

} // namespace

namespace moe {

hipError_t noalloc_scratch(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

} // namespace moe
