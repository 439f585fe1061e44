// gdn_noalloc.hip -- the library-owned scratch buffer behind gdn_forward_noalloc.
//
// gdn_forward_noalloc serves callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the chunked algorithm's scratch space comes from the array below
// instead of a caller workspace.  Every GPU the library runs on holds its own
// copy of the array (zero-initialised when the code object loads) until the
// process ends.  In host code the array's name is only a stand-in for the
// symbol, not a device address: its address on a device is looked up once per
// device with hipGetSymbolAddress, with that device current, and only that
// address is ever handed to kernels.
#include <atomic>
#include <mutex>

#include "gdn_internal.h"

namespace gdn {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_ptr[kMaxDevices];                 // scratch address per device, once looked up
std::atomic<bool> g_have[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!g_have[dev].load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lk(g_lock);
        if (!g_have[dev].load(std::memory_order_relaxed)) {
            void *p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // device `dev` is current
            if (e != hipSuccess) return e;
            g_ptr[dev] = p;
            g_have[dev].store(true, std::memory_order_release);
        }
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gdn
