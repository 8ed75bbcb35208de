// zs_host.cpp -- host part of libzero_shard: shard layout, model-state and
// communication accounting, argument checks, error strings.  No HIP calls.
//
// Layout: "Data parallelism, ZeRO and FSDP", section 2 "What is redundant"
// (rank k owns slice k) and "How FSDP implements ZeRO-3" step 1 (a unit's
// flat parameter cut into N_d equal chunks); padding sits at the tail of the
// flat vector so every slot has the same length S.
// Accounting: the same page's Theorem "ZeRO memory and communication" (table
// and proof); the error convention follows the state_bytes helper of
// "Distributed Training Basics -- DDP and FSDP" (Memory accounting).
#include <cmath>
#include <cstdint>

#include "zs_internal.h"

namespace zs {

static int64_t round_up(int64_t x, int64_t a) { return ((x + a - 1) / a) * a; }

int check_shard(const zs_shard* s)
{
    if (!s) return ZS_ENULL;
    zs_shard ref;
    int rc = zs_layout(s->psi, s->n_d, s->rank, s->align, s->stage, s->out_mode, &ref);
    if (rc != ZS_OK) return rc;
    if (s->shard_len != ref.shard_len || s->shard_offset != ref.shard_offset ||
        s->valid_len != ref.valid_len)
        return ZS_EINVAL_LAYOUT;
    if (s->n_d > ZS_MAX_RANKS) return ZS_EUNSUPPORTED;
    if (s->shard_len % 8 != 0) return ZS_EALIGN;
    return ZS_OK;
}

int check_hparams(const zs_adamw* h)
{
    if (!h) return ZS_ENULL;
    const double v[] = {h->lr, h->beta1, h->beta2, h->eps, h->weight_decay, h->max_grad_norm};
    for (double x : v)
        if (!std::isfinite(x)) return ZS_EINVAL_HPARAM;
    if (h->lr < 0.0) return ZS_EINVAL_HPARAM;
    if (!(h->beta1 >= 0.0 && h->beta1 < 1.0)) return ZS_EINVAL_HPARAM;
    if (!(h->beta2 >= 0.0 && h->beta2 < 1.0)) return ZS_EINVAL_HPARAM;
    if (!(h->eps > 0.0)) return ZS_EINVAL_HPARAM;
    if (h->weight_decay < 0.0) return ZS_EINVAL_HPARAM;
    if (h->step < 1) return ZS_EINVAL_HPARAM;
    return ZS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The section 5 simulator's adamw evaluates 1 - beta and 1 - beta**t in
// double; each scalar is computed in double and rounded to fp32 once.
// A normal, positive power of two (its reciprocal is then exact).
static bool is_pow2f(float x)
{
    if (!(x >= 1.17549435e-38f) || !std::isfinite(x)) return false;
    int e = 0;
    return std::frexp(x, &e) == 0.5f;
}

StepConsts make_consts(const zs_adamw* h)
{
    const double t = static_cast<double>(h->step);
    StepConsts c;
    c.b1 = static_cast<float>(h->beta1);
    c.b2 = static_cast<float>(h->beta2);
    c.c1 = static_cast<float>(1.0 - h->beta1);
    c.c2 = static_cast<float>(1.0 - h->beta2);
    c.bc1 = static_cast<float>(1.0 - std::pow(h->beta1, t));
    c.bc2 = static_cast<float>(1.0 - std::pow(h->beta2, t));
    c.lr = static_cast<float>(h->lr);
    c.wd = static_cast<float>(h->weight_decay);
    c.eps = static_cast<float>(h->eps);
    c.bc1_pow2 = is_pow2f(c.bc1) ? 1 : 0;
    c.bc2_pow2 = is_pow2f(c.bc2) ? 1 : 0;
    c.inv_bc1 = c.bc1_pow2 ? 1.0f / c.bc1 : 0.0f;
    c.inv_bc2 = c.bc2_pow2 ? 1.0f / c.bc2 : 0.0f;
    return c;
}

}  // namespace zs

extern "C" {

int zs_layout(int64_t psi, int32_t n_d, int32_t rank, int64_t align, int32_t stage,
              int32_t out_mode, zs_shard* out)
{
    if (!out) return ZS_ENULL;
    if (psi <= 0) return ZS_EINVAL_PSI;
    if (n_d < 1) return ZS_EINVAL_ND;
    if (rank < 0 || rank >= n_d) return ZS_EINVAL_RANK;
    if (align < 1) return ZS_EINVAL_LAYOUT;
    if (stage < 0 || stage > 3) return ZS_EINVAL_STAGE;
    if (out_mode != ZS_OUT_GATHER && out_mode != ZS_OUT_SHARD) return ZS_EINVAL_STAGE;
    zs_shard s;
    s.psi = psi;
    s.n_d = n_d;
    s.rank = rank;
    s.align = align;
    s.stage = stage;
    s.out_mode = out_mode;
    if (stage == 0) {                    // DDP: the whole vector on every rank
        s.shard_len = zs::round_up(psi, align);
        s.shard_offset = 0;
        s.valid_len = psi;
    } else {
        const int64_t per_rank = psi / n_d + (psi % n_d != 0 ? 1 : 0);
        s.shard_len = zs::round_up(per_rank, align);
        s.shard_offset = static_cast<int64_t>(rank) * s.shard_len;
        const int64_t rest = psi - s.shard_offset;
        s.valid_len = rest <= 0 ? 0 : (rest < s.shard_len ? rest : s.shard_len);
    }
    *out = s;
    return ZS_OK;
}

size_t zs_workspace_bytes(const zs_shard* s)
{
    // One fp64 partial per clip-pass block and one per group of them,
    // rounded up to 256 bytes.
    const int64_t v = (s && s->valid_len > 0) ? s->valid_len : 0;
    const int64_t n = zs::sq_blocks(v);
    const int64_t bytes = (n + zs::sq_groups(n)) * static_cast<int64_t>(sizeof(double));
    return static_cast<size_t>(zs::round_up(bytes > 0 ? bytes : 1, 256));
}

size_t zs_workspace_bytes_units(const zs_shard* s, int32_t units)
{
    // units x (partials + group sums), rounded up to 256 bytes
    if (units < 1) units = 1;
    const int64_t v = (s && s->valid_len > 0) ? s->valid_len : 0;
    const int64_t n = zs::sq_blocks(v);
    const int64_t bytes =
        static_cast<int64_t>(units) * (n + zs::sq_groups(n)) * static_cast<int64_t>(sizeof(double));
    return static_cast<size_t>(zs::round_up(bytes > 0 ? bytes : 1, 256));
}

double zs_state_bytes(double psi, int32_t n_d, int32_t stage, double K)
{
    if (!(psi > 0.0) || n_d < 1) return -1.0;
    const double weights = 2.0 * psi, grads = 2.0 * psi, optim = K * psi;
    switch (stage) {
    case 0: return weights + grads + optim;
    case 1: return weights + grads + optim / n_d;
    case 2: return weights + (grads + optim) / n_d;
    case 3: return (weights + grads + optim) / n_d;
    default: return -1.0;
    }
}

double zs_comm_bytes(double psi, int32_t n_d, int32_t stage, double bytes_per_elem)
{
    if (!(psi > 0.0) || n_d < 1 || stage < 0 || stage > 3) return -1.0;
    // stages 0-2: one reduce-scatter and one all-gather of psi elements;
    // stage 3: a second all-gather for the backward pass.
    const double collectives = stage == 3 ? 3.0 : 2.0;
    return collectives * psi * bytes_per_elem * static_cast<double>(n_d - 1) / n_d;
}

const char* zs_strerror(int code)
{
    switch (code) {
    case ZS_OK: return "ok";
    case ZS_EINVAL_PSI: return "psi must be positive";
    case ZS_EINVAL_ND: return "n_d must be at least 1";
    case ZS_EINVAL_RANK: return "rank must be in [0, n_d)";
    case ZS_EINVAL_LAYOUT: return "align < 1 or shard fields inconsistent with zs_layout";
    case ZS_EALIGN: return "pointer not 16-byte aligned or shard_len not a multiple of 8";
    case ZS_EINVAL_HPARAM: return "invalid AdamW hyperparameter";
    case ZS_EINVAL_STAGE: return "invalid stage or out_mode";
    case ZS_ENULL: return "required pointer is NULL (or both/neither gradient source)";
    case ZS_EUNSUPPORTED: return "n_d exceeds ZS_MAX_RANKS";
    case ZS_EWORKSPACE: return "workspace smaller than zs_workspace_bytes";
    case ZS_ELAUNCH: return "the HIP runtime refused a kernel launch or a set-up call";
    case ZS_EINVAL_REDUCE: return "invalid zs_reduce (dtype, micro-batch index/count or token count)";
    case ZS_EZERO_TOKENS: return "global token count is zero: the update is rejected";
    case ZS_EINVAL_UNITS: return "units must be at least 1";
    case ZS_ESCRATCH: return "shard too large for the static scratch array (ZS_SCRATCH_BYTES)";
    default: return "unknown error";
    }
}

}  // extern "C"
