// zs_kernels.hip -- CDNA4 (gfx950) kernels of the sharded optimizer step and
// the C-ABI entry points that validate arguments and launch them.
//
// Every kernel is a streaming, HBM-bound, elementwise pass (nothing here is
// a contraction, so no MFMA): 64-lane waves, 256-thread blocks, each lane
// owns 8 consecutive parameters per iteration so that every operand moves as
// one 16-byte load or store (8 bf16 = 16 B, 8 fp32 = 2 x 16 B), and a
// grid-stride loop covers shards of any length.  A tail shorter than 8
// elements and the bf16 pads are handled by separate scalar loops.
//
// What is computed ("Data parallelism, ZeRO and FSDP", Lesson 8):
//  - the reduce-scatter's local reduction: the rank gradients are averaged
//    (section 2 "Two GPUs, one batch"; Proposition "DDP is exact"), summed
//    here in rank order in fp32 from the exact widening of bf16, because the
//    order of the sum changes the last bits (the remark after that proof);
//  - the global clip: squared shard norms are summed across shards before
//    the update (section 7 "Common mistakes"), in fp64, in a fixed order;
//  - AdamW, elementwise on the shard (section 2 "What is redundant"), with
//    the expression order of the section 5 simulator's adamw;
//  - the bf16 cast of the new fp32 master shard into the rank's slot of the
//    buffer the all-gather fills (section 2 table "The communication is
//    already there"; "Data parallelism, collectives and ZeRO/FSDP", FSDP
//    diagram: the optimizer returns a new bf16 shard).
//
// Build flags: -ffp-contract=off (no FMA contraction: one rounding per
// written operation), default IEEE division and square root.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "zs_internal.h"

namespace zs {
namespace {

constexpr int kThreads = 256;

// Launch shape (compile-time; a build may override them to sweep):
// blocks in the grid-stride loops, and vectors of 8 parameters each lane
// loads before it computes (more bytes in flight per lane).
#ifndef ZS_STEP_BLOCKS
#define ZS_STEP_BLOCKS 4096
#endif
#ifndef ZS_SQ_BLOCKS
#define ZS_SQ_BLOCKS 4096
#endif
#ifndef ZS_STEP_UNROLL
#define ZS_STEP_UNROLL 1
#endif
#ifndef ZS_SQ_UNROLL
#define ZS_SQ_UNROLL 1
#endif
// Non-temporal (streaming) cache policy for loads / stores of data that is
// touched once per step.
#ifndef ZS_NT_LOAD
#define ZS_NT_LOAD 0
#endif
#ifndef ZS_NT_STORE
#define ZS_NT_STORE 0
#endif
constexpr int kStepMaxBlocks = ZS_STEP_BLOCKS;
constexpr int kSqBlocks = ZS_SQ_BLOCKS;
static_assert(ZS_SQ_BLOCKS <= kMaxSqnormBlocks, "partials must fit the workspace");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SlicePtrs {
    const uint16_t* p[ZS_MAX_RANKS];
};

struct StepArgs {
    SlicePtrs slices;
    const float* mean;
    const double* sqnorm;
    double other_sqnorm;
    double max_norm;
    float* w;
    float* m;
    float* v;
    uint16_t* out;          // slot base: shard element 0
    int64_t valid_len;
    int64_t shard_len;
    int32_t n_d;
    float nd;               // (float)n_d
    float inv_nd;           // 1/n_d, exact when n_d is a power of two
    StepConsts c;
};

struct SqArgs {
    SlicePtrs slices;
    float* mean_out;
    double* partials;
    int64_t valid_len;
    int32_t n_d;
    float nd;
    float inv_nd;
};

// ---- streaming loads and stores -------------------------------------------------

template <typename T>
__device__ __forceinline__ T ld(const T* p)
{
    if constexpr (ZS_NT_LOAD) return __builtin_nontemporal_load(p);
    else return *p;
}

template <typename T>
__device__ __forceinline__ void st(T* p, T v)
{
    if constexpr (ZS_NT_STORE) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---- bf16 --------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even: adding 0x7FFF plus the lowest kept
// bit carries into the kept bits exactly when the dropped half is above one
// half ulp, or equal to it with an odd kept value.  Every NaN becomes the
// canonical 0x7FC0 (the sign of an arithmetic NaN is not defined by IEEE 754
// and differs between processors).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// ---- reduction of the ranks' slices (rank order, fp32) ------------------------

__device__ __forceinline__ void add8(float g[8], u32x4 b)
{
    g[0] = g[0] + bf16_lo(b.x); g[1] = g[1] + bf16_hi(b.x);
    g[2] = g[2] + bf16_lo(b.y); g[3] = g[3] + bf16_hi(b.y);
    g[4] = g[4] + bf16_lo(b.z); g[5] = g[5] + bf16_hi(b.z);
    g[6] = g[6] + bf16_lo(b.w); g[7] = g[7] + bf16_hi(b.w);
}

template <int NDT>
__device__ __forceinline__ float mean_of_sum(float s, float nd, float inv_nd)
{
    // Multiplying by an exact power of two rounds the same exact quotient as
    // dividing by it, so for power-of-two N_d both give the same bits.
    if constexpr (NDT > 0) return s * inv_nd;
    else return s / nd;
}

// Mean of 8 consecutive elements (vector vi) over the ranks, in rank order.
template <int NDT, typename Args>
__device__ __forceinline__ void reduce_vec(const Args& a, int64_t vi, float g[8])
{
    const int nd = NDT > 0 ? NDT : a.n_d;
    const u32x4 x = ld(reinterpret_cast<const u32x4*>(a.slices.p[0]) + vi);
    g[0] = bf16_lo(x.x); g[1] = bf16_hi(x.x);
    g[2] = bf16_lo(x.y); g[3] = bf16_hi(x.y);
    g[4] = bf16_lo(x.z); g[5] = bf16_hi(x.z);
    g[6] = bf16_lo(x.w); g[7] = bf16_hi(x.w);
    // Loads are issued 8 ranks at a time (bounded registers), the additions
    // stay in rank order.
    constexpr int G = 8;
    for (int r0 = 1; r0 < nd; r0 += G) {
        u32x4 b[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (r0 + j < nd) b[j] = ld(reinterpret_cast<const u32x4*>(a.slices.p[r0 + j]) + vi);
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (r0 + j < nd) add8(g, b[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = mean_of_sum<NDT>(g[j], a.nd, a.inv_nd);
}

template <int NDT, typename Args>
__device__ __forceinline__ float reduce_one(const Args& a, int64_t i)
{
    const int nd = NDT > 0 ? NDT : a.n_d;
    float s = __uint_as_float(static_cast<uint32_t>(a.slices.p[0][i]) << 16);
    for (int r = 1; r < nd; ++r)
        s = s + __uint_as_float(static_cast<uint32_t>(a.slices.p[r][i]) << 16);
    return mean_of_sum<NDT>(s, a.nd, a.inv_nd);
}

// ---- AdamW, one element ---------------------------------------------------------

__device__ __forceinline__ void adamw1(const StepConsts& c, float g, float& w, float& m,
                                       float& v)
{
    const float mi = (c.b1 * m) + (c.c1 * g);
    const float vi = (c.b2 * v) + ((c.c2 * g) * g);
    const float mh = mi / c.bc1;
    const float vh = vi / c.bc2;
    const float u = (mh / (sqrtf(vh) + c.eps)) + (c.wd * w);
    w = w - (c.lr * u);
    m = mi;
    v = vi;
}

// min(1, max_norm / (sqrt(Q) + 1e-6)) in double, rounded to fp32; a NaN
// quotient fails the comparison and stays NaN.
__device__ __forceinline__ float clip_coef(double Q, double max_norm)
{
    double c = max_norm / (sqrt(Q) + 1e-6);
    c = (c > 1.0) ? 1.0 : c;
    return static_cast<float>(c);
}

// ---- deterministic fp64 block sum (result valid in thread 0) ------------------

__device__ __forceinline__ double block_sum(double q)
{
    // xor butterfly: both partners add the same two values, so every lane
    // ends with the same bits.
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) q = q + __shfl_xor(q, off, 64);
    __shared__ double wave_sums[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) wave_sums[wave] = q;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) {
        t = wave_sums[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; ++k) t = t + wave_sums[k];
    }
    return t;
}

// ---- kernels ----------------------------------------------------------------------

// Clip pass 1: mean of the slices (optionally stored) and one fp64 partial
// sum of squares per block.  A lane handles vectors vi, vi + stride, ... in
// that order, U of them per iteration (all loads first); the order of its
// fp64 additions does not depend on U.
template <int U, int NDT, bool STORE>
__device__ __forceinline__ void reduce_vectors(const SqArgs& a, int64_t vi, int64_t stride,
                                               double& q)
{
    float g[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) reduce_vec<NDT>(a, vi + u * stride, g[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (STORE) {
            f32x4* o = reinterpret_cast<f32x4*>(a.mean_out) + 2 * (vi + u * stride);
            st(o, f32x4{g[u][0], g[u][1], g[u][2], g[u][3]});
            st(o + 1, f32x4{g[u][4], g[u][5], g[u][6], g[u][7]});
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double d = g[u][j];
            q = q + d * d;
        }
    }
}

template <int NDT, bool STORE>
__global__ void __launch_bounds__(kThreads) k_reduce_sqnorm(const SqArgs a)
{
    constexpr int U = ZS_SQ_UNROLL;
    const int64_t nvec = a.valid_len >> 3;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    double q = 0.0;
    int64_t vi = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (; vi + (U - 1) * stride < nvec; vi += U * stride)
        reduce_vectors<U, NDT, STORE>(a, vi, stride, q);
    for (; vi < nvec; vi += stride) reduce_vectors<1, NDT, STORE>(a, vi, stride, q);
    const int64_t tail0 = nvec * 8;
    if (blockIdx.x == 0 && static_cast<int64_t>(threadIdx.x) < a.valid_len - tail0) {
        const int64_t i = tail0 + threadIdx.x;
        const float g = reduce_one<NDT>(a, i);
        if constexpr (STORE) a.mean_out[i] = g;
        const double d = g;
        q = q + d * d;
    }
    const double t = block_sum(q);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = t;
}

// Clip pass 2: sum the block partials in a fixed order.
__global__ void __launch_bounds__(kThreads)
    k_sqnorm_final(const double* partials, int n, double* out, int accumulate)
{
    double q = 0.0;
    for (int i = threadIdx.x; i < n; i += kThreads) q = q + partials[i];
    const double t = block_sum(q);
    if (threadIdx.x == 0) *out = accumulate ? (*out + t) : t;
}

// The fused step: gradient (mean of the slices, or the stored mean), clip,
// AdamW in place, bf16 cast into the slot, zero pads.  A lane handles U
// vectors (at vi, vi + stride, ...) per iteration, all loads first.
template <int U, bool FROM_SLICES, int NDT, bool CLIP>
__device__ __forceinline__ void step_vectors(const StepArgs& a, const StepConsts& c, float coef,
                                             int64_t vi, int64_t stride)
{
    f32x4* w4 = reinterpret_cast<f32x4*>(a.w);
    f32x4* m4 = reinterpret_cast<f32x4*>(a.m);
    f32x4* v4 = reinterpret_cast<f32x4*>(a.v);
    u32x4* o4 = reinterpret_cast<u32x4*>(a.out);
    float g[U][8], W[U][8], M[U][8], V[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t x = vi + u * stride;
        if constexpr (FROM_SLICES) {
            reduce_vec<NDT>(a, x, g[u]);
        } else {
            const f32x4* g4 = reinterpret_cast<const f32x4*>(a.mean) + 2 * x;
            const f32x4 x0 = ld(g4), x1 = ld(g4 + 1);
            g[u][0] = x0.x; g[u][1] = x0.y; g[u][2] = x0.z; g[u][3] = x0.w;
            g[u][4] = x1.x; g[u][5] = x1.y; g[u][6] = x1.z; g[u][7] = x1.w;
        }
        const f32x4 w0 = ld(w4 + 2 * x), w1 = ld(w4 + 2 * x + 1);
        const f32x4 m0 = ld(m4 + 2 * x), m1 = ld(m4 + 2 * x + 1);
        const f32x4 v0 = ld(v4 + 2 * x), v1 = ld(v4 + 2 * x + 1);
        W[u][0] = w0.x; W[u][1] = w0.y; W[u][2] = w0.z; W[u][3] = w0.w;
        W[u][4] = w1.x; W[u][5] = w1.y; W[u][6] = w1.z; W[u][7] = w1.w;
        M[u][0] = m0.x; M[u][1] = m0.y; M[u][2] = m0.z; M[u][3] = m0.w;
        M[u][4] = m1.x; M[u][5] = m1.y; M[u][6] = m1.z; M[u][7] = m1.w;
        V[u][0] = v0.x; V[u][1] = v0.y; V[u][2] = v0.z; V[u][3] = v0.w;
        V[u][4] = v1.x; V[u][5] = v1.y; V[u][6] = v1.z; V[u][7] = v1.w;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float gj = g[u][j];
            if constexpr (CLIP) gj = gj * coef;
            adamw1(c, gj, W[u][j], M[u][j], V[u][j]);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t x = vi + u * stride;
        st(w4 + 2 * x, f32x4{W[u][0], W[u][1], W[u][2], W[u][3]});
        st(w4 + 2 * x + 1, f32x4{W[u][4], W[u][5], W[u][6], W[u][7]});
        st(m4 + 2 * x, f32x4{M[u][0], M[u][1], M[u][2], M[u][3]});
        st(m4 + 2 * x + 1, f32x4{M[u][4], M[u][5], M[u][6], M[u][7]});
        st(v4 + 2 * x, f32x4{V[u][0], V[u][1], V[u][2], V[u][3]});
        st(v4 + 2 * x + 1, f32x4{V[u][4], V[u][5], V[u][6], V[u][7]});
        st(o4 + x, u32x4{pack_bf16x2(W[u][0], W[u][1]), pack_bf16x2(W[u][2], W[u][3]),
                         pack_bf16x2(W[u][4], W[u][5]), pack_bf16x2(W[u][6], W[u][7])});
    }
}

template <bool FROM_SLICES, int NDT, bool CLIP>
__global__ void __launch_bounds__(kThreads) k_step(const StepArgs a)
{
    // Unrolling multiplies the registers of the slice loads; the bf16-slice
    // source keeps one vector per iteration.
    constexpr int U = FROM_SLICES ? 1 : ZS_STEP_UNROLL;
    float coef = 1.0f;
    if constexpr (CLIP) coef = clip_coef(*a.sqnorm + a.other_sqnorm, a.max_norm);
    const StepConsts c = a.c;
    const int64_t nvec = a.valid_len >> 3;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t gtid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    int64_t vi = gtid;
    for (; vi + (U - 1) * stride < nvec; vi += U * stride)
        step_vectors<U, FROM_SLICES, NDT, CLIP>(a, c, coef, vi, stride);
    for (; vi < nvec; vi += stride) step_vectors<1, FROM_SLICES, NDT, CLIP>(a, c, coef, vi, stride);
    const int64_t tail0 = nvec * 8;
    if (blockIdx.x == 0 && static_cast<int64_t>(threadIdx.x) < a.valid_len - tail0) {
        const int64_t i = tail0 + threadIdx.x;
        float g;
        if constexpr (FROM_SLICES) g = reduce_one<NDT>(a, i);
        else g = a.mean[i];
        if constexpr (CLIP) g = g * coef;
        float w = a.w[i], m = a.m[i], v = a.v[i];
        adamw1(c, g, w, m, v);
        a.w[i] = w;
        a.m[i] = m;
        a.v[i] = v;
        a.out[i] = static_cast<uint16_t>(bf16_rne(w));
    }
    for (int64_t i = a.valid_len + gtid; i < a.shard_len; i += stride) a.out[i] = 0;
}

// Cast and pack only.
__global__ void __launch_bounds__(kThreads)
    k_pack(const float* w, uint16_t* out, int64_t valid_len, int64_t shard_len)
{
    const int64_t nvec = valid_len >> 3;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t gtid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const f32x4* w4 = reinterpret_cast<const f32x4*>(w);
    u32x4* o4 = reinterpret_cast<u32x4*>(out);
    for (int64_t vi = gtid; vi < nvec; vi += stride) {
        const f32x4 a = w4[2 * vi], b = w4[2 * vi + 1];
        o4[vi] = u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                       pack_bf16x2(b.z, b.w)};
    }
    const int64_t tail0 = nvec * 8;
    if (blockIdx.x == 0 && static_cast<int64_t>(threadIdx.x) < valid_len - tail0) {
        const int64_t i = tail0 + threadIdx.x;
        out[i] = static_cast<uint16_t>(bf16_rne(w[i]));
    }
    for (int64_t i = valid_len + gtid; i < shard_len; i += stride) out[i] = 0;
}

// ---- launch helpers -----------------------------------------------------------------

int grid_for(int64_t valid_len, int64_t shard_len, int cap)
{
    const int64_t nvec = valid_len >> 3;
    int64_t blocks = (nvec + kThreads - 1) / kThreads;
    const int64_t pads = shard_len - valid_len;
    const int64_t pad_blocks = (pads + kThreads - 1) / kThreads;
    if (pad_blocks > blocks) blocks = pad_blocks;
    if (blocks < 1) blocks = 1;
    if (blocks > cap) blocks = cap;
    return static_cast<int>(blocks);
}

bool is_pow2(int32_t n) { return n > 0 && (n & (n - 1)) == 0; }

int launched()
{
    return hipGetLastError() == hipSuccess ? ZS_OK : ZS_ELAUNCH;
}

template <int NDT>
void launch_sqnorm_nd(const SqArgs& a, bool store, int blocks, hipStream_t st)
{
    if (store) hipLaunchKernelGGL((k_reduce_sqnorm<NDT, true>), dim3(blocks), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_reduce_sqnorm<NDT, false>), dim3(blocks), dim3(kThreads), 0, st, a);
}

void launch_sqnorm(const SqArgs& a, bool store, int blocks, hipStream_t st)
{
    switch (a.n_d) {
    case 1: launch_sqnorm_nd<1>(a, store, blocks, st); break;
    case 2: launch_sqnorm_nd<2>(a, store, blocks, st); break;
    case 4: launch_sqnorm_nd<4>(a, store, blocks, st); break;
    case 8: launch_sqnorm_nd<8>(a, store, blocks, st); break;
    case 16: launch_sqnorm_nd<16>(a, store, blocks, st); break;
    case 32: launch_sqnorm_nd<32>(a, store, blocks, st); break;
    case 64: launch_sqnorm_nd<64>(a, store, blocks, st); break;
    default: launch_sqnorm_nd<0>(a, store, blocks, st); break;
    }
}

template <bool FROM_SLICES, int NDT>
void launch_step_nd(const StepArgs& a, bool clip, int blocks, hipStream_t st)
{
    if (clip) hipLaunchKernelGGL((k_step<FROM_SLICES, NDT, true>), dim3(blocks), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_step<FROM_SLICES, NDT, false>), dim3(blocks), dim3(kThreads), 0, st, a);
}

void launch_step(const StepArgs& a, bool from_slices, bool clip, int blocks, hipStream_t st)
{
    if (!from_slices) {
        launch_step_nd<false, 0>(a, clip, blocks, st);
        return;
    }
    switch (a.n_d) {
    case 1: launch_step_nd<true, 1>(a, clip, blocks, st); break;
    case 2: launch_step_nd<true, 2>(a, clip, blocks, st); break;
    case 4: launch_step_nd<true, 4>(a, clip, blocks, st); break;
    case 8: launch_step_nd<true, 8>(a, clip, blocks, st); break;
    case 16: launch_step_nd<true, 16>(a, clip, blocks, st); break;
    case 32: launch_step_nd<true, 32>(a, clip, blocks, st); break;
    case 64: launch_step_nd<true, 64>(a, clip, blocks, st); break;
    default: launch_step_nd<true, 0>(a, clip, blocks, st); break;
    }
}

int fill_slices(const zs_shard* s, const uint16_t* const* grad_slices, SlicePtrs* out)
{
    for (int r = 0; r < ZS_MAX_RANKS; ++r) out->p[r] = nullptr;
    if (!grad_slices) return ZS_ENULL;
    for (int r = 0; r < s->n_d; ++r) {
        const uint16_t* p = grad_slices[r];
        if (s->valid_len > 0) {
            if (!p) return ZS_ENULL;
            if (!aligned16(p)) return ZS_EALIGN;
        }
        out->p[r] = p;
    }
    return ZS_OK;
}

uint16_t* slot_base(const zs_shard* s, uint16_t* param_out)
{
    return s->out_mode == ZS_OUT_GATHER ? param_out + s->shard_offset : param_out;
}

}  // namespace
}  // namespace zs

using namespace zs;

extern "C" int shard_grad_sqnorm(const zs_shard* s, const uint16_t* const* grad_slices,
                                 float* mean_out, void* workspace, size_t workspace_bytes,
                                 double* sqnorm_out, int32_t accumulate, void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if (!workspace || !sqnorm_out) return ZS_ENULL;
    if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(sqnorm_out) & 7u) != 0)
        return ZS_EALIGN;
    if (mean_out && !aligned16(mean_out)) return ZS_EALIGN;
    if (workspace_bytes < zs_workspace_bytes(s)) return ZS_EWORKSPACE;
    SqArgs a;
    rc = fill_slices(s, grad_slices, &a.slices);
    if (rc != ZS_OK) return rc;
    a.mean_out = mean_out;
    a.partials = static_cast<double*>(workspace);
    a.valid_len = s->valid_len;
    a.n_d = s->n_d;
    a.nd = static_cast<float>(s->n_d);
    a.inv_nd = is_pow2(s->n_d) ? 1.0f / static_cast<float>(s->n_d) : 0.0f;
    const int blocks = grid_for(s->valid_len, s->valid_len, kSqBlocks);
    (void)hipGetLastError();   // drop an error left by an unrelated earlier call
    hipStream_t st = static_cast<hipStream_t>(stream);
    launch_sqnorm(a, mean_out != nullptr, blocks, st);
    if ((rc = launched()) != ZS_OK) return rc;
    hipLaunchKernelGGL(k_sqnorm_final, dim3(1), dim3(kThreads), 0, st,
                       static_cast<const double*>(workspace), blocks, sqnorm_out,
                       accumulate ? 1 : 0);
    return launched();
}

extern "C" int zero_shard_step(const zs_shard* s, const zs_adamw* h,
                               const uint16_t* const* grad_slices, const float* mean_in,
                               const double* sqnorm, double other_sqnorm, float* master,
                               float* exp_avg, float* exp_avg_sq, uint16_t* param_out,
                               void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if ((rc = check_hparams(h)) != ZS_OK) return rc;
    if ((grad_slices == nullptr) == (mean_in == nullptr)) return ZS_ENULL;
    const bool clip = h->max_grad_norm > 0.0;
    if (clip) {
        if (!sqnorm) return ZS_ENULL;
        if ((reinterpret_cast<uintptr_t>(sqnorm) & 7u) != 0) return ZS_EALIGN;
    }
    if (!param_out) return ZS_ENULL;
    if (!aligned16(param_out)) return ZS_EALIGN;
    if (s->valid_len > 0) {
        if (!master || !exp_avg || !exp_avg_sq) return ZS_ENULL;
        if (!aligned16(master) || !aligned16(exp_avg) || !aligned16(exp_avg_sq))
            return ZS_EALIGN;
        if (mean_in && !aligned16(mean_in)) return ZS_EALIGN;
    }
    StepArgs a;
    if (grad_slices) {
        rc = fill_slices(s, grad_slices, &a.slices);
        if (rc != ZS_OK) return rc;
    } else {
        for (int r = 0; r < ZS_MAX_RANKS; ++r) a.slices.p[r] = nullptr;
    }
    a.mean = mean_in;
    a.sqnorm = sqnorm;
    a.other_sqnorm = other_sqnorm;
    a.max_norm = h->max_grad_norm;
    a.w = master;
    a.m = exp_avg;
    a.v = exp_avg_sq;
    a.out = slot_base(s, param_out);
    a.valid_len = s->valid_len;
    a.shard_len = s->shard_len;
    a.n_d = s->n_d;
    a.nd = static_cast<float>(s->n_d);
    a.inv_nd = is_pow2(s->n_d) ? 1.0f / static_cast<float>(s->n_d) : 0.0f;
    a.c = make_consts(h);
    const int blocks = grid_for(s->valid_len, s->shard_len, kStepMaxBlocks);
    (void)hipGetLastError();
    launch_step(a, grad_slices != nullptr, clip, blocks, static_cast<hipStream_t>(stream));
    return launched();
}

extern "C" int shard_pack_gather(const zs_shard* s, const float* master, uint16_t* param_out,
                                 void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if (!param_out) return ZS_ENULL;
    if (s->valid_len > 0 && !master) return ZS_ENULL;
    if (!aligned16(param_out) || (master && !aligned16(master))) return ZS_EALIGN;
    const int blocks = grid_for(s->valid_len, s->shard_len, kStepMaxBlocks);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_pack, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       master, slot_base(s, param_out), s->valid_len, s->shard_len);
    return launched();
}
