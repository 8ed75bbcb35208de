// zs_kernels.hip -- CDNA4 (gfx950) kernels of the sharded optimizer step,
// their launch shapes, and the enqueue_* functions through which the C-ABI
// entry points (zs_abi.cpp) run them.
//
// Every kernel is a streaming, HBM-bound, elementwise pass (nothing here is
// a contraction, so no MFMA): 64-lane waves, each lane owns 8 parameters and
// moves every operand in 16-byte (or, for bf16 in the contiguous lane
// mapping, 8-byte) vector loads and stores.  Grids are one-shot:
// one thread per 8-parameter vector and hundreds of thousands of blocks,
// dispatched in index order, so the addresses in flight form one window
// that sweeps the arrays front to back (on MI355X a plain copy launched so
// streams at 6.2 TB/s and a read at 6.9 TB/s, where a persistent
// grid-stride loop levels off near 5 TB/s).  The last vector of a shard may
// be partial; it and the bf16 pads are handled element by element by the
// thread that owns it.
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

#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "zs_internal.h"

// Workspace of the allocation-free clip pass (shard_grad_sqnorm_noalloc):
// block partials and group sums, ZS_SCRATCH_BYTES in all.  Each device that
// runs the library holds its own copy until the process ends.  Host code
// reaches a device's copy only through the address static_scratch obtains
// with hipGetSymbolAddress; the name itself is not a device address there.
static __device__ __align__(256) double scratch[ZS_SCRATCH_BYTES / sizeof(double)];

namespace zs {
namespace {

// ---- launch shapes and cache policies ---------------------------------------------
//
// Every choice below was measured on MI355X against its alternatives
// (interleaved repeats in one process, the workloads' real sizes).
//
// Threads per block of the step and the pack (a pack thread owns one
// 8-parameter vector; a step thread 4 or 8 parameters, step_lane_params).
// A streaming step (see kStepStreamBytes) runs one-wave
// blocks: a CU slot frees as soon as its one wave is done, not when the
// slowest wave of a larger block is.  A smaller step, whose operands the
// Infinity Cache partly holds from one step to the next, runs 256-thread
// blocks (15.6M parameters: 72 us, against 78 us in one-wave blocks).
constexpr int step_threads(bool stream) { return stream ? 64 : 256; }
// Parameters one lane of a full block owns.  A streaming step from a stored
// gradient gives each lane 4: one 16-byte vector of every array, so a wave's
// loads and stores are those of a plain copy (see step_per_cu for the
// measurements).  Every other step gives each lane 8: two 16-byte vectors,
// or the 8 bf16 values of each of the N_d gradient slices a fused step
// reduces.
constexpr int step_lane_params(bool stream, bool from_slices)
{
    return (stream && !from_slices) ? 4 : 8;
}
// 8-parameter vectors one block of the step covers.
constexpr int step_vecs(bool stream, bool from_slices)
{
    return step_threads(stream) * step_lane_params(stream, from_slices) / 8;
}
constexpr int kPackThreads = 256;
// Blocks of the step / of the clip pass that may be resident on one CU at a
// time.  A dynamic LDS reservation enforces the cap.  Few resident waves keep
// the window of addresses in flight narrow, which suits the HBM better than a
// full CU when 4 to 65 arrays stream at once.
//  - A streaming step from a stored gradient (4 parameters per lane) runs ten
//    one-wave blocks per CU: 3.92 ms on the 875M-parameter shard, against
//    4.11 ms for the best shape with 8 parameters per lane (six one-wave
//    blocks per CU), 3.92-3.97 at nine and eleven, 4.01-4.04 at eight and
//    twelve, 4.09 at sixteen, 4.19 at 20-24, 4.30 and 4.71 at seven and six,
//    4.51 uncapped; 4.86 against 5.00 ms on the 1.09B shard, 3.92 against
//    4.02 ms for 32 FSDP units.
//  - A streaming step from the slices (8 parameters per lane) runs six
//    one-wave blocks per CU: 4.11 ms on the 875M shard against 4.26 at two
//    256-thread blocks, 4.16 and 4.56 at five and four (its division and
//    square-root chain exposed), 4.15-4.50 at 7-12; 128- or 192-thread blocks
//    and 2 or 4 vectors per thread were slower (these measured on the
//    stored-gradient step before it took 4 parameters per lane).
//  - A smaller step runs two 256-thread blocks per CU.
// The clip pass's shape is sq_shape below.
constexpr int step_per_cu(bool stream, bool from_slices)
{
    return stream ? (from_slices ? 6 : 10) : 2;
}
// Launch shape of the clip pass.  A bf16 reduction of kSqWideNd slices or
// more keeps enough loads in flight per thread to run 512-thread blocks at
// one per CU (64 slices of 1.09B: 24.1 ms, against 25.0 at two per CU, 25.3
// at one 1024-thread block, 27.7-34.1 ms in blocks of 64 to 256 threads);
// fp32 slices, with twice the bytes in flight per thread, run 128-thread
// blocks at two per CU (8 slices of 875M: 5.05 ms, against 5.18 at one
// 256-thread block, 5.13 at four one-wave blocks, 5.23 at three 128-thread
// blocks, 5.44 at two 256-thread blocks, 6.24 at one 128-thread block);
// every other reduction runs 256-thread blocks at two per CU (8 bf16 slices:
// 2.71 ms, against 2.84 ms at two 512-thread blocks; 4 accumulation passes
// 12.72 ms, against 12.91 at one 512-thread block and 14.13 at one 256-thread
// block).  The workspace is sized for the smallest block (kSqThreadsMin).
constexpr int kSqWideNd = 32;
// The wide shape also maps blocks XCD-contiguously (see block_span).
constexpr int kSqWideThreads = 512;
constexpr int kSqThreads = 256;
struct SqShape {
    int threads, per_cu;
};
constexpr SqShape sq_shape(int32_t n_d, bool f32, int acc)
{
    if (f32) return SqShape{kSqThreadsMin, 2};
    return (acc == kAccNone && n_d >= kSqWideNd) ? SqShape{kSqWideThreads, 1}
                                                 : SqShape{kSqThreads, 2};
}
static_assert(kSqThreadsMin % 64 == 0 && kSqThreadsMin < kSqThreads && kSqThreads < kSqWideThreads,
              "three block sizes, the workspace sized for the smallest");
// Gradient slices whose loads one thread has in flight at once; the wide
// specializations (N_d >= kSqWideNd, one block per CU) keep fewer in flight
// (64 slices of 1.09B: 24.04 vs 24.24 ms with 8, 24.75 with 3, 27.5 with 2;
// 8 slices: the same with 4 or 8).
constexpr int kRedGroup = 8;
constexpr int kRedGroupWide = 4;
// Cache-policy words of buffer loads and stores on gfx950: nt (streaming)
// and sc1 (system scope).  Every byte here is touched once per pass.
//  - The clip pass loads and stores nt (plain loads: 3.03 vs 2.80 ms at 8
//    slices, 23.5 vs 22.6 ms at 64; plain stores 3.05 and 23.4 ms).
//  - The step's full blocks store with sc1 and nt when the step streams (see
//    kStepStreamBytes): 4.10 vs 4.30 ms with nt alone on the 875M-parameter
//    shard, 5.18 vs 5.59 ms on the 1.09B one, 4.03 vs 4.17 ms for 32 FSDP
//    units; plain stores were slower still (4.90 vs 4.41 ms at 256-thread
//    blocks).  sc0 on top, or sc1 without nt, gains nothing.  Load policies
//    (nt, sc0, sc1 in any combination) make no difference to either pass.
constexpr int kCpolNt = 2;
constexpr int kCpolSc1Nt = 16 | 2;
// A step that moves at least this many bytes -- twice the 256 MB Infinity
// Cache, so that none of its operands can stay cached from one step to the
// next -- loads all its operands non-temporally (see k_step).  A test build
// lowers it to 0 to run the streaming step on small shards.
#ifndef ZS_STEP_STREAM_BYTES
#define ZS_STEP_STREAM_BYTES (int64_t(512) << 20)
#endif
constexpr int64_t kStepStreamBytes = ZS_STEP_STREAM_BYTES;
// Block-to-data mapping.  Blocks are dispatched round robin over the 8 XCDs.
// Plain: block b takes the b-th span, so neighbouring spans run on
// different XCDs.  XCD-contiguous: the blocks of XCD x (b = x mod 8) take
// one contiguous eighth of the spans.  Measured on MI355X: the clip pass
// over 64 slices is ~3% faster XCD-contiguous (23.0 vs 23.7 ms; 22.4 vs
// 23.1 ms with the contiguous lane mapping), over 8 slices ~3.5% slower; the
// step is within 1% either way, and stays plain.  The clip pass takes it
// with its wide shape (sq_shape).
constexpr int kXcds = 8;

// Logical span of dispatched block b of nb (a bijection on [0, nb)).
__device__ __forceinline__ int64_t block_span(int64_t b, int64_t nb, bool xcd_contiguous)
{
    if (!xcd_contiguous) return b;
    const int64_t q = nb / kXcds, r = nb % kXcds, x = b % kXcds, i = b / kXcds;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Lane mapping of the full blocks of the clip pass and the step: a lane takes
// 4 + 4 elements 256 apart (the contiguous mapping), so every load or store
// instruction of a wave covers one contiguous span (1 KB for fp32, 512 B for
// bf16 read as 8-byte halves), where a lane reading 8 consecutive elements
// (the plain mapping) makes a wave's fp32 access cover 2 KB at a 32-byte
// stride.  Measured on MI355X: contiguous is faster for fp32 slices (6.07 ->
// 5.43 ms, 8 slices of 875M), for 8 bf16 slices (2.93 -> 2.83 ms;
// accumulation passes 13.3 -> 13.0 ms for 4) and, with XCD-contiguous spans,
// for 64 bf16 slices of 1.09B (22.35 vs 22.52 ms).

constexpr int kFinalThreads = 1024;
// Threads of one launch at most.  A dispatch counts its work-items in 32
// bits, so a longer shard takes several launches, each with a grid below
// that (2^31 threads cover 1.7e10 parameters at 8 per thread, 8.6e9 at 4).  A
// test build lowers the limit to run the multi-launch path on small shards.
#ifndef ZS_MAX_LAUNCH_THREADS
#define ZS_MAX_LAUNCH_THREADS (int64_t(1) << 31)
#endif
constexpr int64_t kMaxLaunchThreads = ZS_MAX_LAUNCH_THREADS;
static_assert(kMaxLaunchThreads >= 1024 && kMaxLaunchThreads < (int64_t(1) << 32),
              "a launch holds at least one block of each kernel and fewer than 2^32 threads");
// Blocks of `threads` threads in one launch at most.
constexpr int64_t max_blocks(int threads) { return kMaxLaunchThreads / threads; }
constexpr int kMaxDevices = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT, typename T>
__device__ __forceinline__ T load(const T* p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void store(T* p, T v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// A buffer resource over `bytes` bytes from `base` (uniform across the
// wave), for stores at per-lane byte offsets with an explicit cache-policy
// word (the generic non-temporal hint is lost by the optimizer on some
// float-vector stores, and it has no form for sc1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void* base, uint32_t bytes)
{
    // dword 3: 32-bit data format, as CDNA raw buffer accesses require
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}

template <int CPOL>
__device__ __forceinline__ void buffer_store_f4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v)
{
    const u32x4 b = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(b, r, off, 0, CPOL);
}

template <int CPOL>
__device__ __forceinline__ void buffer_store_u2(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CPOL);
}

template <int CPOL>
__device__ __forceinline__ f32x4 buffer_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL);
    return f32x4{__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z),
                 __uint_as_float(b.w)};
}

template <int CPOL>
__device__ __forceinline__ u32x2 buffer_load_u2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CPOL);
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

// Loading and widening one rank's 8-parameter vector, per element type:
// bf16 (one 16-byte load, widened exactly) or fp32 (two 16-byte loads).
template <typename GT>
struct SliceIO;

template <>
struct SliceIO<uint16_t> {
    using Raw = u32x4;
    template <bool NT>
    __device__ static Raw fetch(const void* p, int64_t vi)
    {
        return load<NT>(reinterpret_cast<const u32x4*>(p) + vi);
    }
    __device__ static void widen(const Raw& b, float v[8])
    {
        v[0] = bf16_lo(b.x); v[1] = bf16_hi(b.x);
        v[2] = bf16_lo(b.y); v[3] = bf16_hi(b.y);
        v[4] = bf16_lo(b.z); v[5] = bf16_hi(b.z);
        v[6] = bf16_lo(b.w); v[7] = bf16_hi(b.w);
    }
    __device__ static float one(const void* p, int64_t i)
    {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
    }
};

template <>
struct SliceIO<float> {
    struct Raw {
        f32x4 a, b;
    };
    template <bool NT>
    __device__ static Raw fetch(const void* p, int64_t vi)
    {
        const f32x4* q = reinterpret_cast<const f32x4*>(p) + 2 * vi;
        return Raw{load<NT>(q), load<NT>(q + 1)};
    }
    __device__ static void widen(const Raw& b, float v[8])
    {
        v[0] = b.a.x; v[1] = b.a.y; v[2] = b.a.z; v[3] = b.a.w;
        v[4] = b.b.x; v[5] = b.b.y; v[6] = b.b.z; v[7] = b.b.w;
    }
    __device__ static float one(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
};

template <int NDT>
__device__ __forceinline__ float mean_of_sum(float s, float nd, float inv_nd)
{
    // Multiplying by an exact power of two rounds the same exact quotient as
    // dividing by it, so for power-of-two N_d both give the same bits.
    if constexpr (NDT > 0) return s * inv_nd;
    else return s / nd;
}

// Reduction of one lane's 8 elements over the ranks, in rank order: the
// mean (sum from rank 0's value, then one division by N_d), or the
// token-weighted sum (((w_0*G_0) + (w_1*G_1)) + ..., every product and sum
// rounded).  `fetch(r)` returns rank r's raw 8 elements; reduce_vec fetches
// the 8 consecutive elements of vector vi.
template <typename GT, int NDT, bool WEIGHTED, typename Fetch, typename Args>
__device__ __forceinline__ void reduce_fetched(const Args& a, Fetch fetch, float g[8])
{
    using IO = SliceIO<GT>;
    const int nd = NDT > 0 ? NDT : a.n_d;
    float v[8];
    IO::widen(fetch(0), v);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if constexpr (WEIGHTED) g[k] = a.wt[0] * v[k];
        else g[k] = v[k];
    }
    // Loads are issued G ranks at a time (bounded registers), the additions
    // stay in rank order.
    constexpr int G = NDT >= kSqWideNd ? kRedGroupWide : kRedGroup;
    for (int r0 = 1; r0 < nd; r0 += G) {
        typename IO::Raw b[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (r0 + j < nd) b[j] = fetch(r0 + j);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (r0 + j < nd) {
                IO::widen(b[j], v);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if constexpr (WEIGHTED) {
                        const float p = a.wt[r0 + j] * v[k];
                        g[k] = g[k] + p;
                    } else {
                        g[k] = g[k] + v[k];
                    }
                }
            }
        }
    }
    if constexpr (!WEIGHTED) {
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = mean_of_sum<NDT>(g[j], a.nd, a.inv_nd);
    }
}

template <typename GT, int NDT, bool WEIGHTED = false, bool NTL = false, typename Args>
__device__ __forceinline__ void reduce_vec(const Args& a, int64_t vi, float g[8])
{
    reduce_fetched<GT, NDT, WEIGHTED>(
        a, [&](int r) { return SliceIO<GT>::template fetch<NTL>(a.slices.p[r], vi); }, g);
}

template <typename GT, int NDT, bool WEIGHTED = false, typename Args>
__device__ __forceinline__ float reduce_one(const Args& a, int64_t i)
{
    using IO = SliceIO<GT>;
    const int nd = NDT > 0 ? NDT : a.n_d;
    float s = IO::one(a.slices.p[0], i);
    if constexpr (WEIGHTED) s = a.wt[0] * s;
    for (int r = 1; r < nd; ++r) {
        const float x = IO::one(a.slices.p[r], i);
        if constexpr (WEIGHTED) {
            const float p = a.wt[r] * x;
            s = s + p;
        } else {
            s = s + x;
        }
    }
    if constexpr (WEIGHTED) return s;
    else return mean_of_sum<NDT>(s, a.nd, a.inv_nd);
}

// Micro-batch accumulation of one reduced value: acc + r, and after the last
// micro-batch (acc + r) / m.
template <int ACC>
__device__ __forceinline__ float accumulate1(const SqArgs& a, float acc, float r)
{
    float x = acc + r;
    if constexpr (ACC == kAccFinal) {
        if (a.inv_micro_count != 0.0f) x = x * a.inv_micro_count;
        else x = x / a.micro_count;
    }
    return x;
}

// ---- AdamW, one element ---------------------------------------------------------

template <bool BC1_POW2 = false, bool BC2_POW2 = false>
__device__ __forceinline__ void adamw1(const StepConsts& c, float g, float& w, float& m,
                                       float& v)
{
    const float mi = (c.b1 * m) + (c.c1 * g);
    const float vi = (c.b2 * v) + ((c.c2 * g) * g);
    const float mh = BC1_POW2 ? mi * c.inv_bc1 : mi / c.bc1;
    const float vh = BC2_POW2 ? vi * c.inv_bc2 : vi / c.bc2;
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

// q + d*d for d widened from fp32: d*d has at most 48 significant bits, so
// it is exact in fp64 and one fused multiply-add rounds exactly as the
// multiply followed by the add.
__device__ __forceinline__ double sq_add(double q, double d) { return __builtin_fma(d, d, q); }

// ---- deterministic fp64 wave and block sums ---------------------------------------

// DPP controls (gfx9 encoding): quad permutations [1,0,3,2] and [2,3,0,1]
// (partners 1 and 2 apart), rotations by 4 and 8 lanes within a row of 16.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// x of another lane by DPP control CTRL (both 32-bit halves moved alike).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x)
{
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, 0xF, 0xF, false));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// x of lane `lane` (uniform).
__device__ __forceinline__ double lane_f64(double x, int lane)
{
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), lane));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), lane));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// The sum of q over the 64 lanes of a full wave, in a fixed order: each quad
// adds partners 1 then 2 apart, each row of 16 adds the quad sums 4 then 8
// lanes on (lane 0 of a row then holds the row's sum), and the rows' sums
// are added in order 0, 1, 2, 3.  The result is uniform.  DPP moves and lane
// reads keep the reduction out of LDS: with the ds_bpermute butterfly of
// __shfl_xor the 8-slice clip pass at 256 threads took 2.78 instead of
// 2.61 ms.
__device__ __forceinline__ double wave_sum(double q)
{
    q = q + dpp_f64<kDppQuadXor1>(q);
    q = q + dpp_f64<kDppQuadXor2>(q);
    q = q + dpp_f64<kDppRowRor4>(q);
    q = q + dpp_f64<kDppRowRor8>(q);
    return ((lane_f64(q, 0) + lane_f64(q, 16)) + lane_f64(q, 32)) + lane_f64(q, 48);
}

// The block's sum of q, valid in thread 0: the wave sums, then wave by wave
// in order.  Every thread of the block must call it.
template <int BS>
__device__ __forceinline__ double block_sum(double q)
{
    q = wave_sum(q);
    __shared__ double wave_sums[BS / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) wave_sums[wave] = q;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) {
        t = wave_sums[0];
#pragma unroll
        for (int k = 1; k < BS / 64; ++k) t = t + wave_sums[k];
    }
    return t;
}

// ---- kernels ----------------------------------------------------------------------

// A full block of BS threads in the contiguous lane mapping (one vector's
// worth of elements per thread); adds the thread's squares to q.  Loads go
// through buffer resources over the block's tile of each slice (and of the
// accumulator), and the reduced values are stored before any square is
// formed: together with the DPP wave sum this took the 8-slice pass at 256
// threads from 2.78 to 2.61 ms (64-bit global loads with the same code: 2.77).
template <typename GT, int NDT, bool STORE, bool WEIGHTED, int ACC, int BS>
__device__ __forceinline__ void reduce_block_contiguous(const SqArgs& a, int64_t base, double& q)
{
    constexpr bool kF32 = std::is_same<GT, float>::value;
    constexpr uint32_t kTile = static_cast<uint32_t>(BS) * 8;       // elements per block
    constexpr int kGBytes = kF32 ? 4 : 2;
    // this lane's two groups of four elements in the block's tile: f32x4
    // index r0 and r0 + 64 (u32x2 index for bf16)
    const uint32_t r0 = (threadIdx.x >> 6) * 128 + (threadIdx.x & 63);
    // the block's tile of the reduced gradient (an accumulator is always stored)
    auto mean_tile = [&]() { return buffer_rsrc(a.mean_out + base * 8, kTile * 4); };
    // the accumulator's loads go first (four accumulation passes over 875M
    // parameters: 12.63 ms, against 12.75 ms with them after the slices')
    f32x4 c0{}, c1{};
    if constexpr (ACC != kAccNone) {
        c0 = buffer_load_f4<kCpolNt>(mean_tile(), r0 * 16);
        c1 = buffer_load_f4<kCpolNt>(mean_tile(), r0 * 16 + 1024);
    }
    float g[8];
    reduce_fetched<GT, NDT, WEIGHTED>(
        a,
        [&](int r) {
            const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(
                const_cast<char*>(static_cast<const char*>(a.slices.p[r])) + base * 8 * kGBytes,
                kTile * kGBytes);
            if constexpr (kF32) {
                return typename SliceIO<float>::Raw{buffer_load_f4<kCpolNt>(sr, r0 * 16),
                                                    buffer_load_f4<kCpolNt>(sr, r0 * 16 + 1024)};
            } else {
                const u32x2 lo = buffer_load_u2<kCpolNt>(sr, r0 * 8);
                const u32x2 hi = buffer_load_u2<kCpolNt>(sr, r0 * 8 + 512);
                return u32x4{lo.x, lo.y, hi.x, hi.y};
            }
        },
        g);
    if constexpr (ACC != kAccNone) {
        const float ac[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = accumulate1<ACC>(a, ac[j], g[j]);
    }
    if constexpr (STORE) {
        buffer_store_f4<kCpolNt>(mean_tile(), r0 * 16, f32x4{g[0], g[1], g[2], g[3]});
        buffer_store_f4<kCpolNt>(mean_tile(), r0 * 16 + 1024, f32x4{g[4], g[5], g[6], g[7]});
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double d = g[j];
        q = sq_add(q, d);
    }
}

// Clip pass 1: the reduced gradient of the slices (optionally stored, or
// accumulated over micro-batches) and one fp64 partial sum of its squares
// per block.  Block span s (see block_span) owns BS consecutive vectors;
// lane l of the block's wave w takes elements 4l..4l+3 and
// 256+4l..256+4l+3 of the wave's 512 (the contiguous lane mapping).  A thread
// adds its squares in a fixed order, and only the last block of a shard,
// which meets the partial vector or runs past valid_len, takes the guarded
// path (vector by vector, then element by element).
template <typename GT, int NDT, bool STORE, bool WEIGHTED, int ACC, int BS>
__global__ void __launch_bounds__(BS) k_reduce_sqnorm(const SqArgs a)
{
    static_assert(STORE || ACC == kAccNone, "an accumulator is always stored");
    static_assert(BS % 64 == 0 && BS >= kSqThreadsMin, "whole waves; workspace sized for the smallest");
    const int64_t nfull = a.valid_len >> 3;
    // the wide shape maps blocks XCD-contiguously (a compile-time choice, so
    // a wave issues its scalar loads without first waiting on a flag)
    const int64_t span = block_span(blockIdx.x, gridDim.x, BS == kSqWideThreads);
    const int64_t base = a.v0 + span * BS;
    double q = 0.0;
    if (base + BS <= nfull) {
        reduce_block_contiguous<GT, NDT, STORE, WEIGHTED, ACC, BS>(a, base, q);
    } else {
        const int64_t vi = base + threadIdx.x;
        if (vi < nfull) {
            float g[8];
            reduce_vec<GT, NDT, WEIGHTED, true>(a, vi, g);
            f32x4* o = reinterpret_cast<f32x4*>(a.mean_out) + 2 * vi;
            if constexpr (ACC != kAccNone) {
                const f32x4 c0 = o[0], c1 = o[1];
                const float ac[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) g[j] = accumulate1<ACC>(a, ac[j], g[j]);
            }
            if constexpr (STORE) {
                store<true>(o, f32x4{g[0], g[1], g[2], g[3]});
                store<true>(o + 1, f32x4{g[4], g[5], g[6], g[7]});
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double d = g[j];
                q = sq_add(q, d);
            }
        } else if (vi == nfull) {
            for (int64_t i = vi * 8; i < a.valid_len; ++i) {
                float g = reduce_one<GT, NDT, WEIGHTED>(a, i);
                if constexpr (ACC != kAccNone) g = accumulate1<ACC>(a, a.mean_out[i], g);
                if constexpr (STORE) a.mean_out[i] = g;
                const double d = g;
                q = sq_add(q, d);
            }
        }
    }
    if (a.partials) {   // uniform: every thread of the block takes the same branch
        const double t = block_sum<BS>(q);
        if (threadIdx.x == 0) a.partials[span] = t;
    }
}

// Clip pass 2: group g of unit u's block partials (n per unit, unit-major),
// [g*kSqGroup, (g+1)*kSqGroup), is summed by block u*ng + g (thread x takes
// x, x + 1024, ... in order; then the block tree).
__global__ void __launch_bounds__(kFinalThreads)
    k_sqnorm_groups(const double* partials, int64_t n, int64_t ng, double* group_sums)
{
    const int64_t u = blockIdx.x / ng, g = blockIdx.x % ng;
    const double* p = partials + u * n;
    const int64_t lo = g * kSqGroup;
    const int64_t hi = lo + kSqGroup < n ? lo + kSqGroup : n;
    double q = 0.0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kFinalThreads) q = q + p[i];
    const double t = block_sum<kFinalThreads>(q);
    if (threadIdx.x == 0) group_sums[blockIdx.x] = t;
}

// Clip pass 3: unit by unit, in unit order, the unit's ng group sums in
// the same fixed order; unit 0's sum replaces *out or is added to it, each
// later unit's sum is added.  This is exactly the sequence of one call per
// unit with accumulate set from the second unit on.
__global__ void __launch_bounds__(kFinalThreads)
    k_sqnorm_final(const double* group_sums, int64_t ng, int32_t units, double* out,
                   int accumulate)
{
    double total = 0.0;
    for (int32_t u = 0; u < units; ++u) {
        double q = 0.0;
        for (int64_t i = threadIdx.x; i < ng; i += kFinalThreads) q = q + group_sums[u * ng + i];
        const double t = block_sum<kFinalThreads>(q);
        if (threadIdx.x == 0) total = u == 0 ? (accumulate ? (*out + t) : t) : (total + t);
        __syncthreads();   // block_sum's LDS is reused by the next unit
    }
    if (threadIdx.x == 0) *out = total;
}

// One element of the step (the partial last vector).
template <bool FROM_SLICES, int NDT, bool CLIP>
__device__ __forceinline__ void step_one(const StepArgs& a, const StepConsts& c, float coef,
                                         int64_t i)
{
    float g;
    if constexpr (FROM_SLICES) g = reduce_one<uint16_t, NDT>(a, i);
    else g = a.mean[i];
    if constexpr (CLIP) g = g * coef;
    float w = a.w[i], m = a.m[i], v = a.v[i];
    adamw1(c, g, w, m, v);
    a.w[i] = w;
    a.m[i] = m;
    a.v[i] = v;
    a.out[i] = static_cast<uint16_t>(bf16_rne(w));
}

// AdamW on a lane's N parameters (clipped gradient when CLIP), bias
// corrections resolved.
template <bool CLIP, bool BC1_POW2, bool BC2_POW2, int N>
__device__ __forceinline__ void adamw_lane(const StepConsts& c, float coef, const float (&g)[N],
                                           float (&W)[N], float (&M)[N], float (&V)[N])
{
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float gj = g[j];
        if constexpr (CLIP) gj = gj * coef;
        adamw1<BC1_POW2, BC2_POW2>(c, gj, W[j], M[j], V[j]);
    }
}

// The arithmetic of one lane's N parameters after its loads: the clip
// coefficient, then AdamW under a uniform branch on this step's bias
// corrections.  The scheduling barriers keep every load ahead of any
// arithmetic, so a wave waits for memory once and computes the fp64 clip
// coefficient while its loads are in flight.
template <bool CLIP, int N>
__device__ __forceinline__ void step_arith(const StepArgs& a, const float (&g)[N], float (&W)[N],
                                           float (&M)[N], float (&V)[N])
{
    __builtin_amdgcn_sched_barrier(0);
    float coef = 1.0f;
    if constexpr (CLIP) coef = clip_coef(*a.sqnorm + a.other_sqnorm, a.max_norm);
    __builtin_amdgcn_sched_barrier(0);
    const StepConsts c = a.c;
    if (c.bc1_pow2) {
        if (c.bc2_pow2) adamw_lane<CLIP, true, true, N>(c, coef, g, W, M, V);
        else adamw_lane<CLIP, true, false, N>(c, coef, g, W, M, V);
    } else {
        if (c.bc2_pow2) adamw_lane<CLIP, false, true, N>(c, coef, g, W, M, V);
        else adamw_lane<CLIP, false, false, N>(c, coef, g, W, M, V);
    }
}

// A full block of the step in the contiguous lane mapping: lane l of wave w
// owns the parameters 4l..4l+3 and 256+4l..256+4l+3 of the wave's 512, i.e.
// the f32x4 groups q0 and q1 = q0 + 64 of the fp32 arrays (and the 8-byte
// groups q0, q1 of the bf16 ones), so every load and store instruction of a
// wave covers one contiguous span.  Stores go through buffer resources over
// the block's tile of each array with the cache-policy word CPOL.
template <bool FROM_SLICES, int NDT, bool CLIP, bool STREAM>
__device__ __forceinline__ void step_block_contiguous(const StepArgs& a, int64_t base)
{
    constexpr int kThreads = step_threads(STREAM);
    static_assert(kThreads % 64 == 0, "whole waves");
    constexpr int CPOL = STREAM ? kCpolSc1Nt : kCpolNt;
    const int64_t r0 = (threadIdx.x >> 6) * 128 + (threadIdx.x & 63);   // in the block's tile
    const int64_t q0 = 2 * base + r0;
    const int64_t q1 = q0 + 64;
    const f32x4* w4 = reinterpret_cast<const f32x4*>(a.w);
    const f32x4* m4 = reinterpret_cast<const f32x4*>(a.m);
    const f32x4* v4 = reinterpret_cast<const f32x4*>(a.v);
    float g[8];
    if constexpr (FROM_SLICES) {
        reduce_fetched<uint16_t, NDT, false>(
            a,
            [&](int r) {
                const u32x2* p = static_cast<const u32x2*>(a.slices.p[r]);
                const u32x2 lo = load<STREAM>(p + q0), hi = load<STREAM>(p + q1);
                return u32x4{lo.x, lo.y, hi.x, hi.y};
            },
            g);
    } else {
        const f32x4* g4 = reinterpret_cast<const f32x4*>(a.mean);
        const f32x4 x0 = load<STREAM>(g4 + q0), x1 = load<STREAM>(g4 + q1);
        g[0] = x0.x; g[1] = x0.y; g[2] = x0.z; g[3] = x0.w;
        g[4] = x1.x; g[5] = x1.y; g[6] = x1.z; g[7] = x1.w;
    }
    const f32x4 w0 = load<STREAM>(w4 + q0), w1 = load<STREAM>(w4 + q1);
    const f32x4 m0 = load<STREAM>(m4 + q0), m1 = load<STREAM>(m4 + q1);
    const f32x4 v0 = load<STREAM>(v4 + q0), v1 = load<STREAM>(v4 + q1);
    float W[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float M[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float V[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    step_arith<CLIP>(a, g, W, M, V);
    // the block's tile: kThreads vectors, 32 bytes each of every fp32 array,
    // half that of the bf16 slot; the lane's byte offsets in it
    constexpr uint32_t kTile = static_cast<uint32_t>(kThreads * 32);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + base * 8, kTile);
    const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(a.m + base * 8, kTile);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(a.v + base * 8, kTile);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(a.out + base * 8, kTile / 2);
    const uint32_t b0 = static_cast<uint32_t>(r0 * 16), b1 = b0 + 64 * 16;
    buffer_store_f4<CPOL>(rw, b0, f32x4{W[0], W[1], W[2], W[3]});
    buffer_store_f4<CPOL>(rw, b1, f32x4{W[4], W[5], W[6], W[7]});
    buffer_store_f4<CPOL>(rm, b0, f32x4{M[0], M[1], M[2], M[3]});
    buffer_store_f4<CPOL>(rm, b1, f32x4{M[4], M[5], M[6], M[7]});
    buffer_store_f4<CPOL>(rv, b0, f32x4{V[0], V[1], V[2], V[3]});
    buffer_store_f4<CPOL>(rv, b1, f32x4{V[4], V[5], V[6], V[7]});
    buffer_store_u2<CPOL>(ro, b0 / 2, u32x2{pack_bf16x2(W[0], W[1]), pack_bf16x2(W[2], W[3])});
    buffer_store_u2<CPOL>(ro, b1 / 2, u32x2{pack_bf16x2(W[4], W[5]), pack_bf16x2(W[6], W[7])});
}

// A full block of the streaming step from a stored gradient: one wave, lane
// l owns the parameters 4l..4l+3 of the block's 256, i.e. the f32x4 group
// q = 2*base + l of every fp32 array and the 8-byte group q of the bf16 slot,
// so every load and store instruction covers one contiguous span (1 KB of an
// fp32 array, 512 bytes of the slot).  Non-temporal loads; stores through
// buffer resources over the block's tile with sc1 and nt.
template <bool CLIP>
__device__ __forceinline__ void step_block_lane4(const StepArgs& a, int64_t base)
{
    static_assert(step_threads(true) == 64 && step_lane_params(true, false) == 4,
                  "one wave, 4 parameters per lane");
    const int64_t q = 2 * base + threadIdx.x;
    const f32x4 x = load<true>(reinterpret_cast<const f32x4*>(a.mean) + q);
    const f32x4 w = load<true>(reinterpret_cast<const f32x4*>(a.w) + q);
    const f32x4 m = load<true>(reinterpret_cast<const f32x4*>(a.m) + q);
    const f32x4 v = load<true>(reinterpret_cast<const f32x4*>(a.v) + q);
    const float g[4] = {x.x, x.y, x.z, x.w};
    float W[4] = {w.x, w.y, w.z, w.w};
    float M[4] = {m.x, m.y, m.z, m.w};
    float V[4] = {v.x, v.y, v.z, v.w};
    step_arith<CLIP>(a, g, W, M, V);
    constexpr uint32_t kTile = 64 * 16;   // bytes of one fp32 array in the block's tile
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.w + base * 8, kTile);
    const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(a.m + base * 8, kTile);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(a.v + base * 8, kTile);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(a.out + base * 8, kTile / 2);
    const uint32_t b = threadIdx.x * 16u;
    buffer_store_f4<kCpolSc1Nt>(rw, b, f32x4{W[0], W[1], W[2], W[3]});
    buffer_store_f4<kCpolSc1Nt>(rm, b, f32x4{M[0], M[1], M[2], M[3]});
    buffer_store_f4<kCpolSc1Nt>(rv, b, f32x4{V[0], V[1], V[2], V[3]});
    buffer_store_u2<kCpolSc1Nt>(ro, b / 2, u32x2{pack_bf16x2(W[0], W[1]), pack_bf16x2(W[2], W[3])});
}

// One full vector vi of the step in the plain mapping (8 consecutive
// parameters; the block that meets valid_len).
template <bool FROM_SLICES, int NDT, bool CLIP, bool STREAM>
__device__ __forceinline__ void step_vector(const StepArgs& a, int64_t vi)
{
    f32x4* w4 = reinterpret_cast<f32x4*>(a.w) + 2 * vi;
    f32x4* m4 = reinterpret_cast<f32x4*>(a.m) + 2 * vi;
    f32x4* v4 = reinterpret_cast<f32x4*>(a.v) + 2 * vi;
    float g[8];
    if constexpr (FROM_SLICES) {
        reduce_vec<uint16_t, NDT, false, STREAM>(a, vi, g);
    } else {
        const f32x4* g4 = reinterpret_cast<const f32x4*>(a.mean) + 2 * vi;
        const f32x4 x0 = load<STREAM>(g4), x1 = load<STREAM>(g4 + 1);
        g[0] = x0.x; g[1] = x0.y; g[2] = x0.z; g[3] = x0.w;
        g[4] = x1.x; g[5] = x1.y; g[6] = x1.z; g[7] = x1.w;
    }
    const f32x4 w0 = load<STREAM>(w4), w1 = load<STREAM>(w4 + 1);
    const f32x4 m0 = load<STREAM>(m4), m1 = load<STREAM>(m4 + 1);
    const f32x4 v0 = load<STREAM>(v4), v1 = load<STREAM>(v4 + 1);
    float W[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float M[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float V[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    step_arith<CLIP>(a, g, W, M, V);
    store<true>(w4, f32x4{W[0], W[1], W[2], W[3]});
    store<true>(w4 + 1, f32x4{W[4], W[5], W[6], W[7]});
    store<true>(m4, f32x4{M[0], M[1], M[2], M[3]});
    store<true>(m4 + 1, f32x4{M[4], M[5], M[6], M[7]});
    store<true>(v4, f32x4{V[0], V[1], V[2], V[3]});
    store<true>(v4 + 1, f32x4{V[4], V[5], V[6], V[7]});
    store<true>(reinterpret_cast<u32x4*>(a.out) + vi,
                u32x4{pack_bf16x2(W[0], W[1]), pack_bf16x2(W[2], W[3]),
                      pack_bf16x2(W[4], W[5]), pack_bf16x2(W[6], W[7])});
}

// The fused step over the slot's shard_len/8 vectors: gradient (mean of the
// slices, or the stored mean), clip, AdamW in place, bf16 cast into the
// slot; vectors past valid_len are pads and get +0.  Block b of a launch
// owns step_vecs(STREAM, FROM_SLICES) consecutive vectors: a streaming step
// from a stored gradient 4 parameters per lane (step_block_lane4), every
// other step 8.
// Full blocks with 8 parameters per lane take the contiguous lane mapping
// (step_block_contiguous): measured against the plain one on MI355X
// (interleaved medians, one box), 4.40 vs 4.47 ms for 875M parameters, 5.33
// vs 5.51 ms for 1.09B, 70 vs 75 us for 15.6M.  The block that meets
// valid_len takes the plain path per vector.
// STREAM: every operand is loaded non-temporally and the full blocks store
// with sc1 as well as nt.  Measured with the contiguous mapping (interleaved
// medians, one box): the stored gradient and v non-temporal, 4.40 vs 4.62 ms
// for 875M parameters, 5.65 vs 5.82 ms for 1.09B, 4.40 vs 4.55 ms for 32
// calls of 27M; w and m as well, 4.32 vs 4.41, 5.57 vs 5.65 and 4.18 vs
// 4.41 ms.  A 15.6M-parameter step, whose 467 MB of operands back-to-back
// steps find partly in the 256 MB Infinity Cache, loses (74 vs 70 us), so
// the host picks STREAM from the bytes the step moves (kStepStreamBytes).
template <bool FROM_SLICES, int NDT, bool CLIP, bool STREAM>
__global__ void __launch_bounds__(step_threads(STREAM)) k_step(const StepArgs a)
{
    const int64_t nfull = a.valid_len >> 3;
    const int64_t nslot = a.shard_len >> 3;
    constexpr int64_t kVecs = step_vecs(STREAM, FROM_SLICES);
    const int64_t base = a.v0 + static_cast<int64_t>(blockIdx.x) * kVecs;
    if (base + kVecs <= nfull) {
        if constexpr (step_lane_params(STREAM, FROM_SLICES) == 4)
            step_block_lane4<CLIP>(a, base);
        else
            step_block_contiguous<FROM_SLICES, NDT, CLIP, STREAM>(a, base);
        return;
    }
    // the block that meets valid_len: one vector per thread, plain mapping
    // (a 4-parameter-per-lane block has more threads than vectors)
    if (threadIdx.x >= kVecs) return;
    const int64_t vi = base + threadIdx.x;
    if (vi < nfull) {
        step_vector<FROM_SLICES, NDT, CLIP, STREAM>(a, vi);
    } else if (vi < nslot) {
        // The partial vector (its valid elements), then pads.
        int64_t i = vi * 8;
        if (i < a.valid_len) {
            float coef = 1.0f;
            if constexpr (CLIP) coef = clip_coef(*a.sqnorm + a.other_sqnorm, a.max_norm);
            for (; i < a.valid_len; ++i) step_one<FROM_SLICES, NDT, CLIP>(a, a.c, coef, i);
        }
        if (i == vi * 8) {
            reinterpret_cast<u32x4*>(a.out)[vi] = u32x4{0u, 0u, 0u, 0u};
        } else {
            for (; i < vi * 8 + 8; ++i) a.out[i] = 0;
        }
    }
}

// Cast and pack only: vector vi of the slot, one per thread.
__global__ void __launch_bounds__(kPackThreads)
    k_pack(const float* w, uint16_t* out, int64_t valid_len, int64_t shard_len, int64_t v0)
{
    const int64_t vi = v0 + static_cast<int64_t>(blockIdx.x) * kPackThreads + threadIdx.x;
    const int64_t nfull = valid_len >> 3;
    if (vi < nfull) {
        const f32x4* w4 = reinterpret_cast<const f32x4*>(w);
        const f32x4 a = w4[2 * vi], b = w4[2 * vi + 1];
        reinterpret_cast<u32x4*>(out)[vi] =
            u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                  pack_bf16x2(b.z, b.w)};
    } else if (vi < (shard_len >> 3)) {
        for (int64_t i = vi * 8; i < vi * 8 + 8; ++i)
            out[i] = i < valid_len ? static_cast<uint16_t>(bf16_rne(w[i])) : uint16_t(0);
    }
}

// ---- launch helpers -----------------------------------------------------------------

int launched()
{
    return hipGetLastError() == hipSuccess ? ZS_OK : ZS_ELAUNCH;
}

// ---- residency cap ----------------------------------------------------------------

// LDS bytes per CU of device `dev` (cached; 160 KB on gfx950).
int device_lds_per_cu(int dev)
{
    static std::atomic<int> cache[kMaxDevices];
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess || v <= 0)
            return -1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Dynamic LDS to request with each launch of kernel K so that at most
// per_cu of its blocks fit on one CU (K itself uses < 1 KB of static LDS).
// per_cu <= 0: no reservation.  The first reservation above the default
// 64 KB per block on a device raises K's limit there, once, to the most any
// launch of K may ask for (one block per CU), because the residency of a
// kernel that serves any N_d (NDT = 0) depends on the call's N_d.
template <auto K>
int lds_reservation(int per_cu, size_t* bytes)
{
    *bytes = 0;
    if (per_cu <= 0) return ZS_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ZS_ELAUNCH;
    const int lds_cu = device_lds_per_cu(dev);
    if (lds_cu <= 0) return ZS_ELAUNCH;
    const int64_t b = (static_cast<int64_t>(lds_cu) / per_cu) / 1024 * 1024 - 1024;
    if (b <= 0) return ZS_OK;
    if (b > 65536) {
        static std::atomic<uint64_t> enabled{0};
        const uint64_t bit = uint64_t(1) << dev;
        if ((enabled.load(std::memory_order_relaxed) & bit) == 0) {
            const int64_t most = static_cast<int64_t>(lds_cu) / 1024 * 1024 - 1024;
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(K),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    static_cast<int>(most)) != hipSuccess)
                return ZS_ELAUNCH;
            enabled.fetch_or(bit, std::memory_order_relaxed);
        }
    }
    *bytes = static_cast<size_t>(b);
    return ZS_OK;
}

// A launch helper called with blocks == kPrepareOnly launches nothing: it
// only makes the per-device set-up calls its kernel needs (prepare_kernels).
constexpr int64_t kPrepareOnly = 0;

template <typename GT, int NDT, bool STORE, bool WEIGHTED, int ACC, int BS>
int launch_reduce_bs(const SqArgs& a, int per_cu, int64_t blocks, hipStream_t st)
{
    size_t lds = 0;
    const int rc = lds_reservation<k_reduce_sqnorm<GT, NDT, STORE, WEIGHTED, ACC, BS>>(per_cu, &lds);
    if (rc != ZS_OK || blocks == kPrepareOnly) return rc;
    hipLaunchKernelGGL((k_reduce_sqnorm<GT, NDT, STORE, WEIGHTED, ACC, BS>), dim3(blocks), dim3(BS),
                       lds, st, a);
    return launched();
}

// The launch shape of sq_shape: fixed for a specialized N_d, chosen per call
// for the generic kernel.
template <typename GT, int NDT, bool STORE, bool WEIGHTED, int ACC>
int launch_reduce_k(const SqArgs& a, int64_t blocks, hipStream_t st)
{
    constexpr bool kF32 = std::is_same<GT, float>::value;
    if constexpr (NDT > 0) {
        constexpr SqShape sh = sq_shape(NDT, kF32, ACC);
        return launch_reduce_bs<GT, NDT, STORE, WEIGHTED, ACC, sh.threads>(a, sh.per_cu, blocks,
                                                                           st);
    } else {
        // the block size the caller sized the grid for: fp32 slices take
        // one shape, bf16 slices one of two
        const SqShape sh = sq_shape(a.n_d, kF32, ACC);
        if constexpr (kF32) {
            if (sh.threads == kSqThreadsMin)
                return launch_reduce_bs<GT, 0, STORE, WEIGHTED, ACC, kSqThreadsMin>(a, sh.per_cu,
                                                                                   blocks, st);
        } else {
            if (sh.threads == kSqWideThreads)
                return launch_reduce_bs<GT, 0, STORE, WEIGHTED, ACC, kSqWideThreads>(
                    a, sh.per_cu, blocks, st);
            if (sh.threads == kSqThreads)
                return launch_reduce_bs<GT, 0, STORE, WEIGHTED, ACC, kSqThreads>(a, sh.per_cu,
                                                                                blocks, st);
        }
        return ZS_ELAUNCH;
    }
}

// The bf16 mean, specialized for the common N_d.
template <int NDT>
int launch_sqnorm_nd(const SqArgs& a, bool store, int64_t blocks, hipStream_t st)
{
    return store ? launch_reduce_k<uint16_t, NDT, true, false, kAccNone>(a, blocks, st)
                 : launch_reduce_k<uint16_t, NDT, false, false, kAccNone>(a, blocks, st);
}

int launch_sqnorm(const SqArgs& a, bool store, int64_t blocks, hipStream_t st)
{
    switch (a.n_d) {
    case 1: return launch_sqnorm_nd<1>(a, store, blocks, st);
    case 2: return launch_sqnorm_nd<2>(a, store, blocks, st);
    case 4: return launch_sqnorm_nd<4>(a, store, blocks, st);
    case 8: return launch_sqnorm_nd<8>(a, store, blocks, st);
    case 16: return launch_sqnorm_nd<16>(a, store, blocks, st);
    case 32: return launch_sqnorm_nd<32>(a, store, blocks, st);
    case 64: return launch_sqnorm_nd<64>(a, store, blocks, st);
    default: return launch_sqnorm_nd<0>(a, store, blocks, st);
    }
}

// Every other reduction (fp32 slices, token weights, accumulation): N_d = 8
// specialized, any other N_d through the generic loop.
template <typename GT, bool WEIGHTED, int ACC>
int launch_reduce_nd(const SqArgs& a, int64_t blocks, hipStream_t st)
{
    if (a.n_d == 8) return launch_reduce_k<GT, 8, true, WEIGHTED, ACC>(a, blocks, st);
    return launch_reduce_k<GT, 0, true, WEIGHTED, ACC>(a, blocks, st);
}

template <typename GT, bool WEIGHTED>
int launch_reduce_acc(const SqArgs& a, int acc, int64_t blocks, hipStream_t st)
{
    switch (acc) {
    case kAccAdd: return launch_reduce_nd<GT, WEIGHTED, kAccAdd>(a, blocks, st);
    case kAccFinal: return launch_reduce_nd<GT, WEIGHTED, kAccFinal>(a, blocks, st);
    default: return launch_reduce_nd<GT, WEIGHTED, kAccNone>(a, blocks, st);
    }
}

int launch_reduce(const SqArgs& a, bool f32, bool weighted, int acc, int64_t blocks,
                  hipStream_t st)
{
    if (!f32 && !weighted && acc == kAccNone) return launch_sqnorm(a, true, blocks, st);
    if (f32)
        return weighted ? launch_reduce_acc<float, true>(a, acc, blocks, st)
                        : launch_reduce_acc<float, false>(a, acc, blocks, st);
    return weighted ? launch_reduce_acc<uint16_t, true>(a, acc, blocks, st)
                    : launch_reduce_acc<uint16_t, false>(a, acc, blocks, st);
}

// The fixed-order sum of the clip pass's block partials (units x blocks,
// unit-major, followed by room for units x groups group sums) into
// *sqnorm_out.
int launch_sqnorm_sums(double* partials, int64_t blocks, int32_t units, double* sqnorm_out,
                       int accumulate, hipStream_t st)
{
    const int64_t groups = sq_groups(blocks);
    double* group_sums = partials + static_cast<int64_t>(units) * blocks;
    if (groups > 0) {
        hipLaunchKernelGGL(k_sqnorm_groups, dim3(static_cast<int64_t>(units) * groups),
                           dim3(kFinalThreads), 0, st, static_cast<const double*>(partials),
                           blocks, groups, group_sums);
        const int rc = launched();
        if (rc != ZS_OK) return rc;
    }
    hipLaunchKernelGGL(k_sqnorm_final, dim3(1), dim3(kFinalThreads), 0, st,
                       static_cast<const double*>(group_sums), groups, units, sqnorm_out,
                       accumulate ? 1 : 0);
    return launched();
}

template <bool FROM_SLICES, int NDT, bool CLIP, bool STREAM>
int launch_step_k(const StepArgs& a, int64_t blocks, hipStream_t st)
{
    size_t lds = 0;
    const int rc =
        lds_reservation<k_step<FROM_SLICES, NDT, CLIP, STREAM>>(step_per_cu(STREAM, FROM_SLICES),
                                                                &lds);
    if (rc != ZS_OK || blocks == kPrepareOnly) return rc;
    hipLaunchKernelGGL((k_step<FROM_SLICES, NDT, CLIP, STREAM>), dim3(blocks),
                       dim3(step_threads(STREAM)), lds, st, a);
    return launched();
}

template <bool FROM_SLICES, int NDT>
int launch_step_nd(const StepArgs& a, bool clip, bool stream, int64_t blocks, hipStream_t st)
{
    if (stream)
        return clip ? launch_step_k<FROM_SLICES, NDT, true, true>(a, blocks, st)
                    : launch_step_k<FROM_SLICES, NDT, false, true>(a, blocks, st);
    return clip ? launch_step_k<FROM_SLICES, NDT, true, false>(a, blocks, st)
                : launch_step_k<FROM_SLICES, NDT, false, false>(a, blocks, st);
}

int launch_step(const StepArgs& a, bool from_slices, bool clip, bool stream, int64_t blocks,
                hipStream_t st)
{
    if (!from_slices) return launch_step_nd<false, 0>(a, clip, stream, blocks, st);
    switch (a.n_d) {
    case 1: return launch_step_nd<true, 1>(a, clip, stream, blocks, st);
    case 2: return launch_step_nd<true, 2>(a, clip, stream, blocks, st);
    case 4: return launch_step_nd<true, 4>(a, clip, stream, blocks, st);
    case 8: return launch_step_nd<true, 8>(a, clip, stream, blocks, st);
    case 16: return launch_step_nd<true, 16>(a, clip, stream, blocks, st);
    case 32: return launch_step_nd<true, 32>(a, clip, stream, blocks, st);
    case 64: return launch_step_nd<true, 64>(a, clip, stream, blocks, st);
    default: return launch_step_nd<true, 0>(a, clip, stream, blocks, st);
    }
}

// Every kernel instantiation the launch helpers above can reach, prepared
// for the current device without a launch (kPrepareOnly): all specialized
// N_d, one power of two and one other N_d through each generic kernel, on
// both sides of the wide clip pass's threshold.
int prepare_kernels()
{
    static const int32_t nds[] = {1, 2, 4, 8, 16, 32, 64, 3, 48};
    for (const int32_t nd : nds) {
        StepArgs sa{};
        sa.n_d = nd;
        SqArgs qa{};
        qa.n_d = nd;
        for (int k = 0; k < 8; ++k) {
            int rc = launch_step(sa, (k & 1) != 0, (k & 2) != 0, (k & 4) != 0, kPrepareOnly,
                                 nullptr);
            if (rc != ZS_OK) return rc;
            if (k < 2 && (rc = launch_sqnorm(qa, k == 1, kPrepareOnly, nullptr)) != ZS_OK)
                return rc;
        }
        for (int k = 0; k < 12; ++k) {
            const int rc = launch_reduce(qa, (k & 1) != 0, (k & 2) != 0, k >> 2, kPrepareOnly,
                                         nullptr);
            if (rc != ZS_OK) return rc;
        }
    }
    return ZS_OK;
}

}  // namespace

// ---- per-device set-up ----------------------------------------------------------------

int static_scratch(void** ptr)
{
    static std::atomic<void*> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ZS_ELAUNCH;
    void* p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ZS_ELAUNCH;
        cache[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return ZS_OK;
}

int prepare_device()
{
    const int rc = prepare_kernels();
    if (rc != ZS_OK) return rc;
    void* p = nullptr;
    return static_scratch(&p);
}

// ---- the passes, as the C-ABI entry points enqueue them -----------------------------

int64_t reduce_blocks(int64_t valid_len, int32_t n_d, bool f32, int acc)
{
    return sq_blocks(valid_len, sq_shape(n_d, f32, acc).threads);
}

int enqueue_reduce(SqArgs a, bool f32, bool weighted, int acc, bool store, double* partials,
                   void* stream)
{
    const bool general = f32 || weighted || acc != kAccNone;
    const SqShape sh = sq_shape(a.n_d, f32, acc);
    const int64_t blocks = sq_blocks(a.valid_len, sh.threads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();   // drop an error left by an unrelated earlier call
    const int64_t cap = max_blocks(sh.threads);
    for (int64_t b0 = 0; b0 < blocks; b0 += cap) {
        const int64_t nb = blocks - b0 < cap ? blocks - b0 : cap;
        a.v0 = b0 * sh.threads;
        a.partials = partials ? partials + b0 : nullptr;
        const int rc = general ? launch_reduce(a, f32, weighted, acc, nb, st)
                               : launch_sqnorm(a, store, nb, st);
        if (rc != ZS_OK) return rc;
    }
    return ZS_OK;
}

int enqueue_sqnorm_sums(double* partials, int64_t blocks, int32_t units, double* sqnorm_out,
                        int accumulate, void* stream)
{
    return launch_sqnorm_sums(partials, blocks, units, sqnorm_out, accumulate,
                              static_cast<hipStream_t>(stream));
}

int enqueue_step(StepArgs a, bool from_slices, bool clip, void* stream)
{
    const int64_t nvec = a.shard_len >> 3;
    // bytes the whole step moves: gradient in, state in and out, bf16 out
    const int64_t step_bytes =
        a.valid_len * (from_slices ? 2 * static_cast<int64_t>(a.n_d) + 26 : 30);
    const bool stream_loads = step_bytes >= kStepStreamBytes;
    const int threads = step_threads(stream_loads);
    const int vecs = step_vecs(stream_loads, from_slices);
    const int64_t blocks = (nvec + vecs - 1) / vecs;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int64_t cap = max_blocks(threads);
    for (int64_t b0 = 0; b0 < blocks; b0 += cap) {
        const int64_t nb = blocks - b0 < cap ? blocks - b0 : cap;
        a.v0 = b0 * vecs;
        const int rc = launch_step(a, from_slices, clip, stream_loads, nb, st);
        if (rc != ZS_OK) return rc;
    }
    return ZS_OK;
}

int enqueue_pack(const float* master, uint16_t* out, int64_t valid_len, int64_t shard_len,
                 void* stream)
{
    const int64_t blocks = ((shard_len >> 3) + kPackThreads - 1) / kPackThreads;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    constexpr int64_t cap = max_blocks(kPackThreads);
    for (int64_t b0 = 0; b0 < blocks; b0 += cap) {
        const int64_t nb = blocks - b0 < cap ? blocks - b0 : cap;
        hipLaunchKernelGGL(k_pack, dim3(nb), dim3(kPackThreads), 0, st, master, out, valid_len,
                           shard_len, b0 * kPackThreads);
        const int rc = launched();
        if (rc != ZS_OK) return rc;
    }
    return ZS_OK;
}

}  // namespace zs
