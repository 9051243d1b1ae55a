// Static device scratch for the entry point that allocates nothing
// (sdpa_math_fwd_noalloc): the key-range workspace of sdpa_math_fwd_ws lives
// in a file-scope device array instead of a caller buffer. Each GPU the
// library runs on holds its own copy of the array until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever handed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "sdpa_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[sdpa::STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace sdpa {

// Device address of the current device's scratch array (looked up on the
// first call per device). Returns a hipError_t as int; *ptr is set on success.
int static_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return (int)hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return 0;
}

}  // namespace sdpa
