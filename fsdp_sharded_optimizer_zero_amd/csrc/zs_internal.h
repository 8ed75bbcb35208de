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

// Number of fp64 partial sums the clip pass writes at most (its grid cap).
constexpr int kMaxSqnormBlocks = 4096;

// Host-side checks; each returns ZS_OK or the error code to report.
int check_shard(const zs_shard* s);
int check_hparams(const zs_adamw* h);
bool aligned16(const void* p);
StepConsts make_consts(const zs_adamw* h);

}  // namespace zs
