// noalloc.hip -- the library-owned scratch of ssm_bwd_noalloc (include/ssm.h), for callers
// that cannot allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The array lives in the code object: every device the library runs on holds its own copy
// from module load until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it asks the runtime for the
// device address once per device and keeps it.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.hpp"

namespace ssm {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // with this device current: its copy of the array (two threads racing here store
        // the same address)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace ssm
