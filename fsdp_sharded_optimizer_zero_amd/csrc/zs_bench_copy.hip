// zs_bench_copy.hip -- kernels used only by the benchmark, not part of the
// ABI: a 16-byte-vector device copy, which gives the practical HBM ceiling
// next to the optimizer kernels and the reference reading of the FETCH_SIZE /
// WRITE_SIZE counters for a kernel whose traffic is known exactly (n16 * 16
// bytes each way); and the step's access pattern without its arithmetic
// (zs_bench_step_pattern, below).
// One vector per thread of a one-shot grid, non-temporal loads, stores with
// the sc1 and nt bits (the streaming step's store policy): the fastest copy
// measured on MI355X (4 GiB each way: 6.60-6.63 TB/s, against 6.44 with nt
// stores alone and 6.20 with plain loads and stores; capping blocks per CU,
// or blocks of 64 to 1024 threads, only slowed it).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over one block's tile (`bytes` from base); accesses past
// it are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}

constexpr int kCpolNt = 2;
constexpr int kSc1Nt = 16 | 2;
constexpr int kCopyThreads = 256;

// Block b copies vectors [b*256, b*256 + 256), then the same span one grid
// further on while any is left (one pass for the one-shot grid the
// benchmark launches).
__global__ void __launch_bounds__(kCopyThreads) k_stream_copy(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, int64_t n16)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads;
    for (int64_t b0 = static_cast<int64_t>(blockIdx.x) * kCopyThreads; b0 < n16; b0 += stride) {
        const int64_t left = n16 - b0;
        const uint32_t bytes = static_cast<uint32_t>((left < kCopyThreads ? left : kCopyThreads) * 16);
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(const_cast<u32x4*>(src + b0), bytes);
        const __amdgpu_buffer_rsrc_t rd = tile_rsrc(dst + b0, bytes);
        if (threadIdx.x < left) {
            const uint32_t off = threadIdx.x * 16u;
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCpolNt);
            __builtin_amdgcn_raw_buffer_store_b128(x, rd, off, 0, kSc1Nt);
        }
    }
}

// src and dst: device, 16-byte aligned, n16 * 16 bytes each, not overlapping.
extern "C" int zs_bench_copy(const void* src, void* dst, int64_t n16, int32_t blocks,
                             void* stream)
{
    if (!src || !dst || n16 < 0 || blocks < 1) return -1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return -5;
    if (n16 == 0) return 0;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_stream_copy, dim3(blocks), dim3(kCopyThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : -11;
}

// The step's memory pattern without its arithmetic: the accesses of a full
// block of the streaming optimizer step from a stored gradient (one wave,
// lane l the f32x4 group l of the block's 256 parameters; non-temporal loads
// of the fp32 gradient, w, m and v; stores of w, m, v and the bf16
// parameters through buffer resources with sc1 and nt), with three additions
// per element in place of AdamW.  The benchmark reports its time next to
// the step's on the same arrays: whether the arithmetic costs the step any
// time.  The bf16 value stored is the high half of w (no rounding).
constexpr int kPatThreads = 64;
constexpr int kPatTile = kPatThreads * 4;   // parameters per block

__global__ void __launch_bounds__(kPatThreads)
    k_step_pattern(const float* __restrict__ g, float* __restrict__ w, float* __restrict__ m,
                   float* __restrict__ v, uint16_t* __restrict__ out)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kPatTile;   // first parameter
    const int64_t q = threadIdx.x;
    const f32x4 g0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + base) + q);
    f32x4 w0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w + base) + q);
    f32x4 m0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(m + base) + q);
    f32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(v + base) + q);
    w0 += g0; m0 += g0; v0 += g0;
    constexpr uint32_t kBytes = kPatTile * 4;
    const uint32_t b0 = static_cast<uint32_t>(q * 16);
    const __amdgpu_buffer_rsrc_t rw = tile_rsrc(w + base, kBytes), rm = tile_rsrc(m + base, kBytes),
                                 rv = tile_rsrc(v + base, kBytes), ro = tile_rsrc(out + base, kBytes / 2);
    auto st4 = [](__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 x) {
        const u32x4 b = {__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z),
                         __float_as_uint(x.w)};
        __builtin_amdgcn_raw_buffer_store_b128(b, r, off, 0, kSc1Nt);
    };
    st4(rw, b0, w0);
    st4(rm, b0, m0);
    st4(rv, b0, v0);
    const u32x2 hi = {(__float_as_uint(w0.x) >> 16) | (__float_as_uint(w0.y) & 0xFFFF0000u),
                      (__float_as_uint(w0.z) >> 16) | (__float_as_uint(w0.w) & 0xFFFF0000u)};
    __builtin_amdgcn_raw_buffer_store_b64(hi, ro, b0 / 2, 0, kSc1Nt);
}

// n parameters (a positive multiple of 256, fewer than 2^31 threads' worth);
// g, w, m, v: device fp32[n], out: device bf16[n], 16-byte aligned.
// per_cu: resident blocks per CU enforced by a dynamic LDS reservation (0:
// no cap).  Returns 0, or -1 (arguments), -5 (alignment), -11 (launch).
extern "C" int zs_bench_step_pattern(const float* g, float* w, float* m, float* v,
                                     uint16_t* out, int64_t n, int32_t per_cu, void* stream)
{
    if (!g || !w || !m || !v || !out || n <= 0 || n % kPatTile != 0 || per_cu < 0) return -1;
    if (n / kPatTile >= (int64_t(1) << 31) / kPatThreads) return -1;
    if ((reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(w) |
         reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v) |
         reinterpret_cast<uintptr_t>(out)) & 15u)
        return -5;
    size_t lds = 0;
    if (per_cu > 0) {
        int dev = 0, lds_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) != hipSuccess || lds_cu <= 2048)
            return -11;
        lds = static_cast<size_t>((lds_cu / per_cu) / 1024 * 1024 - 1024);
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_step_pattern),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                lds_cu / 1024 * 1024 - 1024) != hipSuccess)
            return -11;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_step_pattern, dim3(static_cast<unsigned>(n / kPatTile)),
                       dim3(kPatThreads), lds, static_cast<hipStream_t>(stream), g, w, m, v, out);
    return hipGetLastError() == hipSuccess ? 0 : -11;
}
