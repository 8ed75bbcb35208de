// zs_internal.h -- declarations shared by the host part (zs_host.cpp) and the
// kernel part (zs_kernels.hip) of libzero_shard.  Not part of the ABI.
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

// Launch shape of the clip pass (a build may override it): threads per
// block, and 8-parameter vectors each thread reduces.  The pass writes one
// fp64 partial sum per block into the workspace.
#ifndef ZS_SQ_BS
#define ZS_SQ_BS 512
#endif
#ifndef ZS_SQ_U
#define ZS_SQ_U 1
#endif
constexpr int kSqThreads = ZS_SQ_BS;
constexpr int64_t kSqVecPerBlock = static_cast<int64_t>(ZS_SQ_BS) * ZS_SQ_U;

// Blocks of the clip pass over valid_len parameters: one per kSqVecPerBlock
// vectors of 8 (the last vector may be partial).
inline int64_t sq_blocks(int64_t valid_len)
{
    const int64_t nvec = (valid_len + 7) / 8;
    return (nvec + kSqVecPerBlock - 1) / kSqVecPerBlock;
}

// The block partials are summed in two fixed-order stages: groups of
// kSqGroup partials, then the group sums.
constexpr int64_t kSqGroup = 4096;
inline int64_t sq_groups(int64_t partials) { return (partials + kSqGroup - 1) / kSqGroup; }

// Host-side checks; each returns ZS_OK or the error code to report.
int check_shard(const zs_shard* s);
int check_hparams(const zs_adamw* h);
bool aligned16(const void* p);
StepConsts make_consts(const zs_adamw* h);

}  // namespace zs
