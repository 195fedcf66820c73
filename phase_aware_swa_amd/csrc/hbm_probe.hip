// hbm_probe.hip -- plain streaming kernels that measure what HBM delivers on
// this GPU (read only, and read + write), for the benchmark's practical
// ceilings.  Built into its own library (libhbmprobe.so); the attention
// library does not use it.
//
// Each lane moves 16-byte chunks; a workgroup of 256 lanes walks the buffer
// grid-stride, U chunks per lane per iteration with all U loads issued
// before any is used.  The read kernel folds what it loads into an XOR that
// is stored only if it equals a constant (so the loads stay live).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[blockIdx.x * 256 + threadIdx.x] = acc.x;
}

template <int U>
__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                   int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + u * 256);
    }
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16 * 256 * unroll) from src; sink must hold
// grid * 256 uint32 values.  unroll: 4, 8 or 16.  Returns a hipError_t.
int hbm_probe_read(const void* src, int64_t bytes, void* sink, int unroll, int grid, void* stream)
{
    const int64_t n16 = bytes / 16;
    if (bytes % (16 * 256 * (int64_t)unroll) || grid < 1) return (int)hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(256);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* p = (const u32x4*)src;
    uint32_t* k = (uint32_t*)sink;
    if (unroll == 4) hipLaunchKernelGGL(read_kernel<4>, g, b, 0, s, p, n16, k);
    else if (unroll == 8) hipLaunchKernelGGL(read_kernel<8>, g, b, 0, s, p, n16, k);
    else if (unroll == 16) hipLaunchKernelGGL(read_kernel<16>, g, b, 0, s, p, n16, k);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16 * 256 * unroll) from src to dst.
int hbm_probe_copy(void* dst, const void* src, int64_t bytes, int unroll, int grid, void* stream)
{
    const int64_t n16 = bytes / 16;
    if (bytes % (16 * 256 * (int64_t)unroll) || grid < 1) return (int)hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(256);
    hipStream_t s = (hipStream_t)stream;
    u32x4* d = (u32x4*)dst;
    const u32x4* p = (const u32x4*)src;
    if (unroll == 4) hipLaunchKernelGGL(copy_kernel<4>, g, b, 0, s, d, p, n16);
    else if (unroll == 8) hipLaunchKernelGGL(copy_kernel<8>, g, b, 0, s, d, p, n16);
    else if (unroll == 16) hipLaunchKernelGGL(copy_kernel<16>, g, b, 0, s, d, p, n16);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // extern "C"
