// zs_internal.h -- declarations shared by the host parts (zs_host.cpp,
// zs_abi.cpp) and the kernel part (zs_kernels.hip) of libzero_shard.  Not
// part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "zero_shard.h"

namespace zs {

// fp32 scalars of one AdamW step, each rounded once from double.
struct StepConsts {
    float b1, b2, c1, c2, bc1, bc2, lr, wd, eps;
    // When bc1 (bc2) is a power of two, x / bc equals x * (1 / bc) bit for
    // bit (both are the rounding of the same exact value), and the kernel
    // multiplies by the exact reciprocal instead of dividing.
    float inv_bc1, inv_bc2;
    int32_t bc1_pow2, bc2_pow2;
};

// The clip pass runs blocks of 128, 256 or 512 threads (one 8-parameter
// vector per thread, the size chosen per call by the kernel part) and writes
// one fp64 partial sum per block into the workspace; the workspace is sized
// for the smallest block.
constexpr int kSqThreadsMin = 128;

// Blocks of the clip pass over valid_len parameters at `threads` threads per
// block (the last vector may be partial).
inline int64_t sq_blocks(int64_t valid_len, int threads = kSqThreadsMin)
{
    const int64_t nvec = (valid_len + 7) / 8;
    return (nvec + threads - 1) / threads;
}

// The block partials are summed in two fixed-order stages: groups of
// kSqGroup partials, then the group sums.
constexpr int64_t kSqGroup = 4096;
inline int64_t sq_groups(int64_t partials) { return (partials + kSqGroup - 1) / kSqGroup; }

struct SlicePtrs {
    const void* p[ZS_MAX_RANKS];   // bf16 or fp32 rows, by the kernel's element type
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
    int64_t v0;             // first vector of this launch
    int32_t n_d;
    float nd;               // (float)n_d
    float inv_nd;           // 1/n_d, exact when n_d is a power of two
    StepConsts c;
};

struct SqArgs {
    SlicePtrs slices;
    float wt[ZS_MAX_RANKS]; // token weights (weighted reduction only)
    float* mean_out;        // the reduced gradient; also read in place when
                            // it is a micro-batch accumulator
    double* partials;       // one per block of this launch; null: no norm
    int64_t valid_len;
    int64_t v0;             // first vector of this launch
    int32_t n_d;
    float nd;
    float inv_nd;
    float micro_count;      // m, the divisor of the last micro-batch
    float inv_micro_count;  // 1/m when m is a power of two (exact), else 0
};

// What the clip pass does with the accumulator: write the reduced slice
// (no accumulation, or the first micro-batch), add it to the accumulator,
// or add it and divide by the micro-batch count (the last micro-batch).
enum AccMode { kAccNone = 0, kAccAdd = 1, kAccFinal = 2 };

// The passes (zs_kernels.hip).  Each enqueues its launches on `stream` (a
// hipStream_t), splitting a grid longer than one launch may hold, and
// returns ZS_OK or ZS_ELAUNCH; arguments are validated by the caller.
//   reduce_blocks: the number of blocks (fp64 partials) the clip pass runs
//     over valid_len parameters for this reduction (at most
//     sq_blocks(valid_len)).
//   enqueue_reduce: the clip pass / general reduction over a.valid_len
//     (a.v0 and a.partials are set per launch; partials: reduce_blocks(...)
//     fp64 slots, or null for no norm).  f32/weighted/acc select the general
//     reduction (always stored); otherwise bf16 rank-order mean, stored iff
//     `store`.
//   enqueue_sqnorm_sums: units x blocks partials (unit-major) -> *sqnorm_out
//     (added to it if accumulate), in a fixed order.
//   enqueue_step: the fused AdamW step over a.shard_len (a.v0 set per launch).
//   enqueue_pack: bf16 cast of master[0, valid_len) and +0 pads into out.
int64_t reduce_blocks(int64_t valid_len, int32_t n_d, bool f32, int acc);
int enqueue_reduce(SqArgs a, bool f32, bool weighted, int acc, bool store, double* partials,
                   void* stream);
int enqueue_sqnorm_sums(double* partials, int64_t blocks, int32_t units, double* sqnorm_out,
                        int accumulate, void* stream);
int enqueue_step(StepArgs a, bool from_slices, bool clip, void* stream);
int enqueue_pack(const float* master, uint16_t* out, int64_t valid_len, int64_t shard_len,
                 void* stream);

// Per-device set-up (zs_kernels.hip), for the current device; each returns
// ZS_OK or ZS_ELAUNCH.
//   prepare_device: the set-up calls every kernel launch needs (the LDS
//     query and the kernels' dynamic-LDS limits) and the address of the
//     static scratch array, so that later calls make none.
//   static_scratch: *ptr = this device's ZS_SCRATCH_BYTES scratch array.
int prepare_device();
int static_scratch(void** ptr);

// Host-side checks; each returns ZS_OK or the error code to report.
int check_shard(const zs_shard* s);
int check_hparams(const zs_adamw* h);
bool aligned16(const void* p);
StepConsts make_consts(const zs_adamw* h);

}  // namespace zs
