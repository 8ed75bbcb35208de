// zsg_device.hip -- GPU side of the seeded input generator (definition in
// zsg_def.h): fills device buffers in place so that multi-GB inputs never
// cross PCIe.  Produces the same bits as zsg_host.c (checked by a GPU test).
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define ZSG_FN __host__ __device__ static inline
#include "zsg_def.h"

#define ZSG_DEV_FSQRT(x) sqrtf(x)

namespace {

struct GenArgs {
    uint64_t key, key_mask, key_val;
    double sigma, p_out, sigma_out;
    int absval;
    int is_bf16;
    int64_t start, n;
    void* out;
};

__device__ inline double value_at(const GenArgs& a, int64_t i, double z)
{
    double x = z * a.sigma;
    if (a.p_out > 0.0) {
        uint64_t h = zsg_draw(a.key_mask, (uint64_t)i);
        double u = (double)(h >> 11) * (1.0 / 9007199254740992.0);
        if (u < a.p_out) {
            double w0, w1;
            ZSG_NORMAL_PAIR(a.key_val, (uint64_t)i >> 1, w0, w1, ZSG_DEV_FSQRT);
            x = ((i & 1) ? w1 : w0) * a.sigma_out;
        }
    }
    if (a.absval && x < 0.0) x = -x;
    return x;
}

__device__ inline void store(const GenArgs& a, int64_t pos, double x)
{
    if (a.is_bf16)
        static_cast<uint16_t*>(a.out)[pos] = zsg_trunc_bf16(x);
    else
        static_cast<uint32_t*>(a.out)[pos] = zsg_trunc_f32(x);
}

__global__ void __launch_bounds__(256) k_fill(GenArgs a)
{
    const int64_t end = a.start + a.n;
    const int64_t j0 = a.start >> 1;
    const int64_t j1 = (end - 1) >> 1;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = j0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j <= j1; j += stride) {
        double z0, z1;
        ZSG_NORMAL_PAIR(a.key, (uint64_t)j, z0, z1, ZSG_DEV_FSQRT);
        int64_t e0 = 2 * j, e1 = e0 + 1;
        if (e0 >= a.start && e0 < end) store(a, e0 - a.start, value_at(a, e0, z0));
        if (e1 >= a.start && e1 < end) store(a, e1 - a.start, value_at(a, e1, z1));
    }
}

int launch(GenArgs a, hipStream_t stream)
{
    if (a.n <= 0) return 0;
    if (a.start < 0 || !a.out) return -1;
    int64_t pairs = ((a.start + a.n - 1) >> 1) - (a.start >> 1) + 1;
    int64_t blocks = (pairs + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

GenArgs make(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
             double sigma, int absval, double p_out, double sigma_out)
{
    GenArgs a;
    a.key = zsg_key(seed, stream, rank, step);
    a.key_mask = zsg_key(seed, stream | ZSG_SUBSTREAM_MASK, rank, step);
    a.key_val = zsg_key(seed, stream | ZSG_SUBSTREAM_OUTLIER, rank, step);
    a.sigma = sigma;
    a.p_out = p_out;
    a.sigma_out = sigma_out;
    a.absval = absval;
    a.is_bf16 = 0;
    a.start = 0;
    a.n = 0;
    a.out = nullptr;
    return a;
}

}  // namespace

extern "C" int zsg_dev_fill_f32(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
                                double sigma, int absval, int64_t start, int64_t n,
                                float* out, void* hip_stream)
{
    GenArgs a = make(seed, stream, rank, step, sigma, absval, 0.0, 0.0);
    a.start = start;
    a.n = n;
    a.out = out;
    return launch(a, static_cast<hipStream_t>(hip_stream));
}

extern "C" int zsg_dev_fill_bf16(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
                                 double sigma, double p_out, double sigma_out, int64_t start,
                                 int64_t n, uint16_t* out, void* hip_stream)
{
    GenArgs a = make(seed, stream, rank, step, sigma, 0, p_out, sigma_out);
    a.is_bf16 = 1;
    a.start = start;
    a.n = n;
    a.out = out;
    return launch(a, static_cast<hipStream_t>(hip_stream));
}
