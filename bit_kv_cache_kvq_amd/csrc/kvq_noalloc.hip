// kvq_noalloc.hip -- the device-resident workspace of kvq_decode_attn_noalloc: one array per
// GPU, held until the process ends, whose device address is looked up once per device.
#include <atomic>
#include <mutex>

#include "kvq_internal.h"

// The scratch array.  In host code its name is only a host-side stand-in: kernels get the
// device address from hipGetSymbolAddress (per device), never the name itself.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace kvq {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

} // namespace

hipError_t noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        // first call on this device (it is current): its copy of the array's address
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return e != hipSuccess ? e : hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

} // namespace kvq
