// zs_bench_copy.hip -- a 16-byte-vector device copy, used only by the
// benchmark: it gives the practical HBM ceiling next to the optimizer
// kernels, and the reference reading of the FETCH_SIZE / WRITE_SIZE counters
// for a kernel whose traffic is known exactly (n16 * 16 bytes each way).
// Non-temporal loads and stores, one vector per thread of a one-shot grid:
// the fastest copy measured on MI355X (4 GiB each way: 6.49 TB/s, against
// 6.20 with plain loads and stores; capping blocks per CU only slowed it).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_stream_copy(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int64_t n16)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// src and dst: device, 16-byte aligned, n16 * 16 bytes each, not overlapping.
extern "C" int zs_bench_copy(const void* src, void* dst, int64_t n16, int32_t blocks,
                             void* stream)
{
    if (!src || !dst || n16 < 0 || blocks < 1) return -1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return -5;
    if (n16 == 0) return 0;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_stream_copy, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : -11;
}
