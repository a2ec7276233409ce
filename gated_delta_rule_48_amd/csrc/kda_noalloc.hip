// Scratch memory of the allocation-free chunked forward
// (kda_chunk_fwd_noalloc): a static device array, one copy on every GPU the
// library runs on, held until the process ends.  In host code the array's
// name is only a host-side stand-in; its device address on a GPU comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept in a per-device table.  Only that address is ever handed to kernels.
#include <atomic>
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

namespace kda {

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace kda
