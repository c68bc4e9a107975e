// kda_scratch.hip -- the library's static device scratch: the Tb / P rows that
// the prefill's prep kernel writes and its state kernel reads, for the entry
// point that allocates nothing (kda_chunk_fwd_noalloc).  Every GPU the library
// runs on holds one copy from the code object's load until the process ends.
//
// In host code `scratch` is only a handle for hipGetSymbolAddress, never a
// device address: the kernels get the per-device address that lookup returns.
#include <mutex>

#include "kda_launch.h"

static __device__ __align__(256) unsigned char scratch[kda::kScratchBytes];

namespace kda {
namespace {
std::mutex g_mu;
void *g_ptr[kScratchMaxDevices];   // per device, set by the first lookup there
}  // namespace

hipError_t scratch_address(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
