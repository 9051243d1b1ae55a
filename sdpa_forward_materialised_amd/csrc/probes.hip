// Streaming fill and copy kernels (measurement references, see sdpa_probe.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void fill_kernel(u32x4* __restrict__ dst, size_t n, uint32_t value) {
    const u32x4 v = {value, value, value, value};
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        __builtin_nontemporal_store(v, dst + i);
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// 256 CUs x 8 workgroups of 256 threads keeps every CU busy.
constexpr int kGrid = 2048;

}  // namespace

extern "C" int sdpa_probe_fill(void* dst, size_t bytes, uint32_t value, void* stream) {
    if (!dst || bytes % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return (int)hipErrorInvalidValue;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(fill_kernel, dim3(kGrid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<u32x4*>(dst), bytes / 16, value);
    return (int)hipGetLastError();
}

extern "C" int sdpa_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || bytes % 16 || reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(src) % 16)
        return (int)hipErrorInvalidValue;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(copy_kernel, dim3(kGrid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), bytes / 16);
    return (int)hipGetLastError();
}
