// zs_abi.cpp -- the C-ABI entry points that run the passes: argument
// validation (nothing is enqueued when a call is rejected), the scalars each
// pass needs, and the calls into the kernel part (enqueue_*, zs_kernels.hip).
// No HIP calls here.
//
// What each entry point computes is stated with its declaration in
// zero_shard.h, with the passage of "Data parallelism, ZeRO and FSDP" (and
// its companion pages) that defines it.
#include <cstdint>

#include "zs_internal.h"

namespace zs {
namespace {

bool is_pow2(int32_t n) { return n > 0 && (n & (n - 1)) == 0; }

// The n_d slice pointers of one unit into the kernel arguments; each must be
// non-null and 16-byte aligned unless the shard is empty.
int fill_slices(const zs_shard* s, const void* const* grad_slices, SlicePtrs* out)
{
    for (int r = 0; r < ZS_MAX_RANKS; ++r) out->p[r] = nullptr;
    if (!grad_slices) return ZS_ENULL;
    for (int r = 0; r < s->n_d; ++r) {
        const void* p = grad_slices[r];
        if (s->valid_len > 0) {
            if (!p) return ZS_ENULL;
            if (!aligned16(p)) return ZS_EALIGN;
        }
        out->p[r] = p;
    }
    return ZS_OK;
}

// Where the shard's bf16 values go: its slot of the gather buffer, or the
// rank's own shard buffer.
uint16_t* slot_base(const zs_shard* s, uint16_t* param_out)
{
    return s->out_mode == ZS_OUT_GATHER ? param_out + s->shard_offset : param_out;
}

bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// The reduction's scalars for n_d ranks and m micro-batches (no weights).
SqArgs reduce_args(const zs_shard* s, float* grad_out, int32_t micro_count)
{
    SqArgs a{};
    a.mean_out = grad_out;
    a.valid_len = s->valid_len;
    a.n_d = s->n_d;
    a.nd = static_cast<float>(s->n_d);
    a.inv_nd = is_pow2(s->n_d) ? 1.0f / static_cast<float>(s->n_d) : 0.0f;
    a.micro_count = static_cast<float>(micro_count);
    a.inv_micro_count = is_pow2(micro_count) ? 1.0f / static_cast<float>(micro_count) : 0.0f;
    return a;
}

}  // namespace
}  // namespace zs

using namespace zs;

namespace zs {
namespace {

// The clip pass of one shard into the partials workspace `partials`; the
// shard, sqnorm_out and mean_out have been checked.
int sqnorm_pass(const zs_shard* s, const uint16_t* const* grad_slices, float* mean_out,
                double* partials, double* sqnorm_out, int32_t accumulate, void* stream)
{
    SqArgs a = reduce_args(s, mean_out, 1);
    int rc = fill_slices(s, reinterpret_cast<const void* const*>(grad_slices), &a.slices);
    if (rc != ZS_OK) return rc;
    rc = enqueue_reduce(a, false, false, kAccNone, mean_out != nullptr, partials, stream);
    if (rc != ZS_OK) return rc;
    return enqueue_sqnorm_sums(partials, reduce_blocks(s->valid_len, s->n_d, false, kAccNone), 1,
                               sqnorm_out, accumulate, stream);
}

}  // namespace
}  // namespace zs

extern "C" int zs_init(void) { return prepare_device(); }

extern "C" int shard_grad_sqnorm(const zs_shard* s, const uint16_t* const* grad_slices,
                                 float* mean_out, void* workspace, size_t workspace_bytes,
                                 double* sqnorm_out, int32_t accumulate, void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if (!workspace || !sqnorm_out) return ZS_ENULL;
    if (!aligned16(workspace) || !aligned8(sqnorm_out)) return ZS_EALIGN;
    if (mean_out && !aligned16(mean_out)) return ZS_EALIGN;
    if (workspace_bytes < zs_workspace_bytes(s)) return ZS_EWORKSPACE;
    return sqnorm_pass(s, grad_slices, mean_out, static_cast<double*>(workspace), sqnorm_out,
                       accumulate, stream);
}

extern "C" int shard_grad_sqnorm_noalloc(const zs_shard* s, const uint16_t* const* grad_slices,
                                         float* mean_out, double* sqnorm_out,
                                         int32_t accumulate, void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if (!sqnorm_out) return ZS_ENULL;
    if (!aligned8(sqnorm_out)) return ZS_EALIGN;
    if (mean_out && !aligned16(mean_out)) return ZS_EALIGN;
    if (zs_workspace_bytes(s) > ZS_SCRATCH_BYTES) return ZS_ESCRATCH;
    SqArgs tmp;
    rc = fill_slices(s, reinterpret_cast<const void* const*>(grad_slices), &tmp.slices);
    if (rc != ZS_OK) return rc;
    void* ws = nullptr;
    if ((rc = static_scratch(&ws)) != ZS_OK) return rc;
    return sqnorm_pass(s, grad_slices, mean_out, static_cast<double*>(ws), sqnorm_out,
                       accumulate, stream);
}

extern "C" int shard_grad_sqnorm_units(const zs_shard* s, int32_t units,
                                       const uint16_t* const* grad_slices,
                                       float* const* mean_out, void* workspace,
                                       size_t workspace_bytes, double* sqnorm_out,
                                       int32_t accumulate, void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if (units < 1) return ZS_EINVAL_UNITS;
    if (!grad_slices || !workspace || !sqnorm_out) return ZS_ENULL;
    if (!aligned16(workspace) || !aligned8(sqnorm_out)) return ZS_EALIGN;
    if (workspace_bytes < zs_workspace_bytes_units(s, units)) return ZS_EWORKSPACE;
    // validate every unit before enqueueing anything
    for (int32_t u = 0; u < units; ++u) {
        SlicePtrs tmp;
        rc = fill_slices(s, reinterpret_cast<const void* const*>(grad_slices + u * s->n_d), &tmp);
        if (rc != ZS_OK) return rc;
        if (mean_out && mean_out[u] && !aligned16(mean_out[u])) return ZS_EALIGN;
    }
    const int64_t blocks = reduce_blocks(s->valid_len, s->n_d, false, kAccNone);
    double* partials = static_cast<double*>(workspace);
    for (int32_t u = 0; u < units; ++u) {
        SqArgs a = reduce_args(s, mean_out ? mean_out[u] : nullptr, 1);
        fill_slices(s, reinterpret_cast<const void* const*>(grad_slices + u * s->n_d), &a.slices);
        rc = enqueue_reduce(a, false, false, kAccNone, a.mean_out != nullptr,
                            partials + static_cast<int64_t>(u) * blocks, stream);
        if (rc != ZS_OK) return rc;
    }
    return enqueue_sqnorm_sums(partials, blocks, units, sqnorm_out, accumulate, stream);
}

extern "C" int shard_grad_reduce(const zs_shard* s, const zs_reduce* r,
                                 const void* const* grad_slices, float* grad_out,
                                 void* workspace, size_t workspace_bytes, double* sqnorm_out,
                                 int32_t accumulate, void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if (!r) return ZS_ENULL;
    if ((r->grad_dtype != ZS_GRAD_BF16 && r->grad_dtype != ZS_GRAD_F32) || r->reserved != 0 ||
        r->micro_count < 1 || r->micro < 0 || r->micro >= r->micro_count)
        return ZS_EINVAL_REDUCE;
    if (s->valid_len > 0 && !grad_out) return ZS_ENULL;
    if (grad_out && !aligned16(grad_out)) return ZS_EALIGN;
    if (sqnorm_out) {
        if (!workspace) return ZS_ENULL;
        if (!aligned16(workspace) || !aligned8(sqnorm_out)) return ZS_EALIGN;
        if (workspace_bytes < zs_workspace_bytes(s)) return ZS_EWORKSPACE;
    }
    SqArgs a = reduce_args(s, grad_out, r->micro_count);
    rc = fill_slices(s, grad_slices, &a.slices);
    if (rc != ZS_OK) return rc;
    const bool weighted = r->rank_tokens != nullptr;
    if (weighted) {
        // w_r = n_r / T in double, rounded once; T = 0 rejects the update.
        double T = 0.0;
        for (int k = 0; k < s->n_d; ++k) {
            if (r->rank_tokens[k] < 0) return ZS_EINVAL_REDUCE;
            T += static_cast<double>(r->rank_tokens[k]);
        }
        if (T == 0.0) return ZS_EZERO_TOKENS;
        for (int k = 0; k < s->n_d; ++k)
            a.wt[k] = static_cast<float>(static_cast<double>(r->rank_tokens[k]) / T);
    }
    const int acc = r->micro == 0 ? kAccNone
                  : (r->micro == r->micro_count - 1 ? kAccFinal : kAccAdd);
    double* partials = sqnorm_out ? static_cast<double*>(workspace) : nullptr;
    const bool f32 = r->grad_dtype == ZS_GRAD_F32;
    rc = enqueue_reduce(a, f32, weighted, acc, true, partials, stream);
    if (rc != ZS_OK || !sqnorm_out) return rc;
    return enqueue_sqnorm_sums(partials, reduce_blocks(s->valid_len, s->n_d, f32, acc), 1,
                               sqnorm_out, accumulate, stream);
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
        // a sum of squares is never negative; NaN and +Inf propagate
        if (other_sqnorm < 0.0) return ZS_EINVAL_HPARAM;
        if (!sqnorm) return ZS_ENULL;
        if (!aligned8(sqnorm)) return ZS_EALIGN;
    }
    if (!param_out) return ZS_ENULL;
    if (!aligned16(param_out)) return ZS_EALIGN;
    if (s->valid_len > 0) {
        if (!master || !exp_avg || !exp_avg_sq) return ZS_ENULL;
        if (!aligned16(master) || !aligned16(exp_avg) || !aligned16(exp_avg_sq))
            return ZS_EALIGN;
        if (mean_in && !aligned16(mean_in)) return ZS_EALIGN;
    }
    StepArgs a{};
    if (grad_slices) {
        rc = fill_slices(s, reinterpret_cast<const void* const*>(grad_slices), &a.slices);
        if (rc != ZS_OK) return rc;
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
    return enqueue_step(a, grad_slices != nullptr, clip, stream);
}

extern "C" int shard_pack_gather(const zs_shard* s, const float* master, uint16_t* param_out,
                                 void* stream)
{
    int rc = check_shard(s);
    if (rc != ZS_OK) return rc;
    if (!param_out) return ZS_ENULL;
    if (s->valid_len > 0 && !master) return ZS_ENULL;
    if (!aligned16(param_out) || (master && !aligned16(master))) return ZS_EALIGN;
    return enqueue_pack(master, slot_base(s, param_out), s->valid_len, s->shard_len, stream);
}
