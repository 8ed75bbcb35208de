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

// Host-side checks; each returns ZS_OK or the error code to report.
int check_shard(const zs_shard* s);
int check_hparams(const zs_adamw* h);
bool aligned16(const void* p);
StepConsts make_consts(const zs_adamw* h);

}  // namespace zs
