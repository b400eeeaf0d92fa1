// kda_scratch.hip -- the library's static device scratch, for the entry
// point that allocates nothing (kda_prefill_cp_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, allocated when the code object is loaded on that device and
// kept until the process ends.  Host code never uses the array's name as an
// address (on the host it names a stand-in, not device memory): the device
// address is taken once per device with hipGetSymbolAddress, with that device
// current, and cached here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>

#include "kda.h"

static_assert(KDA_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of its alignment");

__device__ __align__(256) unsigned char scratch[KDA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device id
}  // namespace

// Device address and size of the current device's scratch.  The first call on
// a device resolves the address (with that device current, as every call into
// the library runs); later calls read the cached value.  Concurrent first
// calls resolve the same address and store the same value.
extern "C" hipError_t kda_static_scratch(void **ptr, size_t *bytes)
{
    *ptr = nullptr;
    *bytes = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    *bytes = KDA_STATIC_SCRATCH_BYTES;
    return hipSuccess;
}
