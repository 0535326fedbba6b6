// noalloc.hip -- device scratch of the allocation-free attention entry point.
//
// csa2_sparse_swa_attn_noalloc is csa2_sparse_swa_attn for callers that
// cannot allocate device memory: the per-unit partials of its split pass go
// to this file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy of the array (CSA2_ATTN_SCRATCH_BYTES)
// from the time the library's code is loaded on it until the process ends.
//
// In host code the array's name is not a device address, so it is never
// passed to a kernel: its address on the current device is looked up once per
// device with hipGetSymbolAddress and kept, and that pointer is what the
// launches receive.
#include <atomic>
#include <mutex>

#include "../../include/csa2.h"
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

static __device__ __align__(256) uint8_t scratch[CSA2_ATTN_SCRATCH_BYTES];

constexpr int NA_MAX_DEVICES = 64;
static std::atomic<void*> g_scratch_ptr[NA_MAX_DEVICES];
static std::mutex g_scratch_mu;

hipError_t noalloc_scratch(void** out, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= NA_MAX_DEVICES) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // with `dev` current: the address of this device's copy
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    *bytes = CSA2_ATTN_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace csa2
