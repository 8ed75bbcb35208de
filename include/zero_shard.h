/*
 * zero_shard.h -- C ABI of the MI355X sharded optimizer step.
 *
 * One GPU's share of the ZeRO-1/2/3 and FSDP optimizer step: the local
 * reduction of the reduce-scatter (N_d ranks' bf16 gradient slices of this
 * rank's shard into an fp32 mean), the squared gradient norm for a global
 * clip, the elementwise mixed-precision AdamW update of the shard's fp32
 * master weights and moments, and the bf16 cast and pack of the new shard
 * into the buffer the all-gather fills.
 *
 * Sources (page title, then section):
 *  - "Data parallelism, ZeRO and FSDP" (ML Systems, Lesson 8): section 2
 *    "What is redundant" (AdamW is elementwise, so rank k owns and updates
 *    slice k) and "The communication is already there" (reduce-scatter, the
 *    update of slice k, then the all-gather of the new weights); section 3
 *    Theorem "ZeRO memory and communication" (12 optimizer bytes per
 *    parameter, the stages); "How FSDP implements ZeRO-3" step 1 (a unit's
 *    flat parameter cut into N_d equal chunks) and step 4 (a normal
 *    optimizer on the local shards); section 5 "In code" (the adamw of the
 *    simulator, whose expression order this library follows); section 7
 *    "Common mistakes" (a global clip needs the squared shard norms summed).
 *  - "Distributed Training Basics -- DDP and FSDP": the clip at the update
 *    boundary in its DDP reference program; the errors raised by its
 *    state_bytes helper.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers (HBM of the current HIP device),
 *    16-byte aligned, owned by the caller.  The library allocates nothing at
 *    run time.  The only state it keeps is, per device, the LDS size it
 *    queried, the kernels' dynamic-LDS limits it raised and the address of its
 *    static scratch array (see shard_grad_sqnorm_noalloc), all set once,
 *    thread-safely, by zs_init or by the first call that needs them; calls
 *    may come from several host threads at once.
 *  - HIP graphs: every entry point enqueues kernels only (no memset, no
 *    allocation, no synchronisation), so its calls may be captured into a
 *    HIP graph.  The per-device set-up above is not a stream operation and
 *    must not happen inside a capture: call zs_init on each device (or make
 *    one call of each kind eagerly) before capturing.
 *  - bf16 values are passed as their uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Calls only enqueue
 *    work and return; results are ready after the caller synchronises the
 *    stream.  A device fault surfaces at that synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; a call
 *    that returns an error other than ZS_ELAUNCH has enqueued nothing and
 *    written nothing.  ZS_ELAUNCH reports a launch the runtime refused; the
 *    call's earlier launches (a long shard takes several) may have run.
 *  - Return value: ZS_OK (0) or one of the negative codes below.  Nothing is
 *    thrown across the ABI.
 *  - Arithmetic: IEEE-754 fp32, round to nearest even, no fused
 *    multiply-add, correctly rounded division and square root, subnormals
 *    kept; the squared norm in fp64.  NaN and Inf propagate (no skipping).
 *  - Outputs must not overlap inputs, except master/exp_avg/exp_avg_sq which
 *    are updated in place.  Calls that write the same buffers must not run
 *    concurrently on different streams.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define ZS_OK               0
#define ZS_EINVAL_PSI     (-1)   /* psi <= 0 */
#define ZS_EINVAL_ND      (-2)   /* n_d < 1 */
#define ZS_EINVAL_RANK    (-3)   /* rank outside [0, n_d) */
#define ZS_EINVAL_LAYOUT  (-4)   /* align < 1, or shard_len / shard_offset /
                                    valid_len not those zs_layout gives */
#define ZS_EALIGN         (-5)   /* a pointer not 16-byte aligned, or
                                    shard_len not a multiple of 8 */
#define ZS_EINVAL_HPARAM  (-6)   /* lr < 0, beta outside [0,1), eps <= 0,
                                    weight_decay < 0, step < 1, or any
                                    hyperparameter not finite */
#define ZS_EINVAL_STAGE   (-7)   /* stage outside 0..3 or unknown out_mode */
#define ZS_ENULL          (-8)   /* a required pointer is NULL, or both /
                                    neither of grad_slices and mean_in */
#define ZS_EUNSUPPORTED   (-9)   /* n_d > ZS_MAX_RANKS */
#define ZS_EWORKSPACE    (-10)   /* workspace smaller than zs_workspace_bytes */
#define ZS_ELAUNCH       (-11)   /* the HIP runtime rejected a kernel launch
                                    or a set-up call (device query, kernel
                                    attribute, symbol address) */
#define ZS_EINVAL_REDUCE (-12)   /* zs_reduce: unknown grad_dtype, reserved != 0,
                                    micro outside [0, micro_count), micro_count
                                    < 1, or a negative token count */
#define ZS_EZERO_TOKENS  (-13)   /* every rank_tokens entry is 0: the update is
                                    rejected on every rank; nothing is written */
#define ZS_EINVAL_UNITS  (-14)   /* units < 1 */
#define ZS_ESCRATCH      (-15)   /* shard_grad_sqnorm_noalloc: the shard needs
                                    more than ZS_SCRATCH_BYTES of workspace */

#define ZS_MAX_RANKS 64          /* gradient slices one call can reduce */
/* Bytes of the per-device static scratch array of shard_grad_sqnorm_noalloc:
 * the workspace of shards of up to 2,146,959,360 parameters. */
#define ZS_SCRATCH_BYTES ((size_t)16 << 20)

/* Where the new bf16 shard goes. */
#define ZS_OUT_GATHER 0  /* param_out is the bf16[n_d * shard_len] all-gather
                            buffer; this rank writes at shard_offset (stage 0:
                            offset 0, the whole vector) */
#define ZS_OUT_SHARD  1  /* param_out is this rank's own bf16[shard_len] */

/* One rank's shard of a flat parameter vector of psi elements.
 * Stages: 0 = DDP (nothing sharded: the rank owns the whole vector),
 * 1 = ZeRO-1, 2 = ZeRO-2, 3 = ZeRO-3 / FSDP.  The stage does not change the
 * arithmetic, only the layout (stage 0) and which out_mode is natural. */
typedef struct zs_shard {
    int64_t psi;           /* parameters in the flat vector (or FSDP unit) */
    int32_t n_d;           /* data-parallel ranks */
    int32_t rank;          /* k, the owner of this shard */
    int64_t align;         /* shard_len is a multiple of this */
    int64_t shard_len;     /* S: padded slice length */
    int64_t shard_offset;  /* k*S (0 at stage 0) */
    int64_t valid_len;     /* V = clamp(psi - k*S, 0, S): real parameters */
    int32_t stage;         /* 0..3 */
    int32_t out_mode;      /* ZS_OUT_GATHER or ZS_OUT_SHARD */
} zs_shard;

/* AdamW hyperparameters (decoupled weight decay inside the step, on every
 * element), in double; rounded once to fp32 by the library. */
typedef struct zs_adamw {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;          /* t >= 1, the bias-correction step; the caller
                              increments it between calls */
    double max_grad_norm;  /* > 0: clip the gradient to this global L2 norm;
                              <= 0: no clip */
} zs_adamw;

/* Fill *out with the shard of `rank`.  "Data parallelism, ZeRO and FSDP",
 * section 2 "What is redundant" (GPU k owns slice k of the parameters) and
 * "How FSDP implements ZeRO-3" step 1 (FSDP1 cuts a unit's flat parameter
 * into N_d equal chunks).  The flat vector is padded at its tail
 * to n_d*S with S = roundup(ceil(psi/n_d), align) (stage 0: S =
 * roundup(psi, align), offset 0, valid_len psi); slot k is [k*S, (k+1)*S).
 * Host only.  Errors: ZS_EINVAL_PSI/ND/RANK/LAYOUT(align < 1)/STAGE,
 * ZS_ENULL (out). */
int zs_layout(int64_t psi, int32_t n_d, int32_t rank, int64_t align, int32_t stage,
              int32_t out_mode, zs_shard* out);

/* Bytes of device workspace shard_grad_sqnorm needs for the squared norm of
 * "Data parallelism, ZeRO and FSDP", section 7 "Common mistakes" (global
 * clipping of sharded gradients): one fp64 partial sum
 * per block of its first pass (at most one block per 1024 parameters) plus
 * one per group of 4096 such partials, rounded up to 256 bytes -- 6.8 MB for
 * an 875M-parameter shard, at least 256 bytes (an empty shard).  Host only. */
size_t zs_workspace_bytes(const zs_shard* s);

/* Model-state bytes per GPU of the table of "Data parallelism, ZeRO and
 * FSDP", section 3, Theorem "ZeRO memory and communication" (the same
 * factors as state_bytes in "Distributed Training Basics -- DDP and FSDP",
 * "Memory accounting", whose argument checks this follows): weights and gradients
 * 2 bytes each, K optimizer bytes per parameter.  stage 0: (4+K)psi,
 * 1: 4psi + K psi/n_d, 2: 2psi + (2+K) psi/n_d, 3: (4+K) psi/n_d.
 * Returns -1 for psi <= 0, n_d < 1 or an unknown stage.  Host only. */
double zs_state_bytes(double psi, int32_t n_d, int32_t stage, double K);

/* Bytes each GPU sends per step, from the elements column of the same
 * Theorem ("Data parallelism, ZeRO and FSDP", section 3, proof items 5-7):
 * 2psi elements for stages 0-2, 3psi for
 * stage 3, times bytes_per_elem and (n_d-1)/n_d (ring collectives).
 * Returns -1 on invalid arguments.  Host only. */
double zs_comm_bytes(double psi, int32_t n_d, int32_t stage, double bytes_per_elem);

/* Clip pass: the reduce-scatter's local reduction plus this shard's squared
 * L2 norm.  "Data parallelism, ZeRO and FSDP": section 2 "The communication
 * is already there" (after the reduce-scatter GPU k holds slice k of the
 * gradients) with the averaging of section 2 "Two GPUs, one batch" and the
 * Proposition "DDP is exact" (the mean of the ranks' gradients; its order of
 * summation changes only the last bits, hence the fixed rank order here);
 * section 7 "Common mistakes" (a global clip over sharded gradients sums the
 * squared shard norms, which this call provides for this shard).
 *   grad_slices  host array of n_d device pointers; grad_slices[r] is rank
 *                r's bf16 gradient for this shard, valid_len elements.
 *   mean_out     device fp32[valid_len] or NULL.  If given, receives
 *                g_i = (sum over r = 0..n_d-1 in rank order of the widened
 *                bf16 values) / n_d.
 *   workspace    device, >= zs_workspace_bytes(s) bytes, 16-byte aligned;
 *                contents on entry are ignored.
 *   sqnorm_out   device, one double: sum of (double)g_i^2 over the shard.
 *                accumulate == 0 overwrites it; accumulate != 0 adds the
 *                shard's value to it (for a norm over several FSDP units,
 *                summed in call order).
 * The fp64 sum is taken in a fixed tree order (run-to-run deterministic for
 * one shape), not in ascending element order.  An empty shard (valid_len 0)
 * contributes 0.  Errors: ZS_ENULL, ZS_EINVAL_*, ZS_EALIGN, ZS_EUNSUPPORTED,
 * ZS_EWORKSPACE, ZS_ELAUNCH. */
int shard_grad_sqnorm(const zs_shard* s, const uint16_t* const* grad_slices, float* mean_out,
                      void* workspace, size_t workspace_bytes, double* sqnorm_out,
                      int32_t accumulate, void* stream);

/* Bytes of device workspace shard_grad_sqnorm_units needs for `units`
 * units of layout s: units x what one shard needs (6.8 MB per 875M
 * parameters of a unit).  Host only. */
size_t zs_workspace_bytes_units(const zs_shard* s, int32_t units);

/* The clip pass of `units` FSDP units that share one layout (e.g. identical
 * transformer blocks), as one call: the same result, bit for bit, as
 * shard_grad_sqnorm on unit 0 with `accumulate` followed by
 * shard_grad_sqnorm on units 1.. with accumulate = 1 -- the global squared
 * norm over the units ("Data parallelism, ZeRO and FSDP", section 7: the
 * norm of sharded gradients sums the squared shard norms), each unit's sum
 * taken in the fixed per-shard order and added in unit order -- but with
 * two partial-sum kernels in all instead of two per unit.
 *   grad_slices  host array of units x n_d device pointers, unit-major
 *                (unit u's rank r slice at [u*n_d + r]).
 *   mean_out     NULL, or a host array of `units` device pointers (each
 *                fp32[valid_len] or NULL) receiving each unit's mean.
 *   workspace    >= zs_workspace_bytes_units(s, units) bytes.
 * Errors: as shard_grad_sqnorm, plus ZS_EINVAL_UNITS; every unit's
 * pointers are checked before anything is enqueued. */
int shard_grad_sqnorm_units(const zs_shard* s, int32_t units, const uint16_t* const* grad_slices,
                            float* const* mean_out, void* workspace, size_t workspace_bytes,
                            double* sqnorm_out, int32_t accumulate, void* stream);

/* Element type of the gradient slices a reduction reads. */
#define ZS_GRAD_BF16 0   /* bf16, widened exactly to fp32 */
#define ZS_GRAD_F32  1   /* fp32 (the reduce_dtype=float32 policy) */

/* How shard_grad_reduce combines the ranks' slices and the micro-batches. */
typedef struct zs_reduce {
    int32_t grad_dtype;          /* ZS_GRAD_BF16 or ZS_GRAD_F32, every slice */
    int32_t micro;               /* j, this micro-batch: 0 <= j < micro_count */
    int32_t micro_count;         /* m >= 1 micro-batches per optimizer step
                                    (1: no gradient accumulation) */
    int32_t reserved;            /* must be 0 */
    const int64_t* rank_tokens;  /* NULL: the mean over ranks; else a host
                                    array of n_d valid-token counts, and the
                                    ranks are weighted by n_r / T */
} zs_reduce;

/* The general clip pass: reduces the ranks' slices of one micro-batch and
 * accumulates micro-batches into the shard's fp32 gradient.
 *   "Data parallelism, ZeRO and FSDP", section 3 "Gradient accumulation"
 *   (ZeRO-2 reduce-scatters after every micro-batch) and section 6 (Llama 3
 *   reduce-scattered gradients in fp32); "Distributed Training Basics --
 *   DDP and FSDP", "DDP: replicated state, partitioned examples" (weight
 *   ranks by valid tokens; a zero global count rejects the update) and
 *   "Accumulation, clipping and scaling measurements" (clip and step at the
 *   effective-update boundary).
 * Per element i < valid_len, in fp32:
 *   r_i = the mean over ranks, as shard_grad_sqnorm computes it, of bf16 or
 *         fp32 slices; or, with rank_tokens, ((w_0*G_0[i]) + (w_1*G_1[i]))
 *         + ... in rank order, w_r = f32(n_r / T) computed in double,
 *         T = sum of n_r, every product and sum rounded;
 *   micro == 0:                grad_out[i] = r_i
 *   0 < micro < m - 1:         grad_out[i] = grad_out[i] + r_i
 *   micro == m - 1 > 0:        grad_out[i] = (grad_out[i] + r_i) / m
 * so after the last micro-batch grad_out holds the step's gradient, the
 * mean over micro-batches, ready for zero_shard_step's mean_in.
 *   grad_slices  host array of n_d device pointers, each to valid_len
 *                elements of grad_dtype, 16-byte aligned.
 *   grad_out     device fp32[valid_len], 16-byte aligned; read and written
 *                in place for micro > 0.
 *   workspace, sqnorm_out, accumulate: as for shard_grad_sqnorm, applied to
 *                the values written.  sqnorm_out may be NULL (then no norm
 *                and no workspace are needed), e.g. before the last
 *                micro-batch.
 * Errors: ZS_ENULL, ZS_EINVAL_*, ZS_EINVAL_REDUCE, ZS_EZERO_TOKENS (nothing
 * enqueued), ZS_EALIGN, ZS_EUNSUPPORTED, ZS_EWORKSPACE, ZS_ELAUNCH. */
int shard_grad_reduce(const zs_shard* s, const zs_reduce* r, const void* const* grad_slices,
                      float* grad_out, void* workspace, size_t workspace_bytes,
                      double* sqnorm_out, int32_t accumulate, void* stream);

/* The fused optimizer step of this shard.  "Data parallelism, ZeRO and
 * FSDP": section 2 "What is redundant" (AdamW is elementwise, so GPU k
 * updates slice k from that slice's gradient, moments and fp32 master
 * weights alone) and the table of "The communication is already there" (the
 * update sits between the reduce-scatter and the all-gather of the new
 * weights); section 3 Theorem (K = 12 bytes of fp32 master weight, m and v
 * per parameter); section 5 "In code" (the AdamW expression order below);
 * section 7 "Common mistakes" (the clip uses the global norm).  Exactly one
 * gradient source:
 *   grad_slices  host array of n_d device pointers to bf16[valid_len]
 *                (reduced here, in rank order, as shard_grad_sqnorm does), or
 *   mean_in      device fp32[valid_len], the mean from shard_grad_sqnorm.
 * If h->max_grad_norm > 0: `sqnorm` (device, one double, this shard's or the
 * accumulated squared norm) is required and the global squared norm is
 * Q = *sqnorm + other_sqnorm (other_sqnorm stands for the scalar all-reduce
 * of the other ranks' squared shard norms; a negative value is rejected with
 * ZS_EINVAL_HPARAM, NaN and +Inf propagate as IEEE arithmetic does);
 * coef = f32(min(1, max_grad_norm / (sqrt(Q) + 1e-6))) in double, NaN kept,
 * and g = g * coef.  Otherwise `sqnorm` and other_sqnorm are ignored.
 * Then, for i < valid_len, in this order and in fp32 (b1 = f32(beta1),
 * c1 = f32(1 - beta1), bc1 = f32(1 - beta1^t), likewise b2, c2, bc2):
 *   m' = (b1*m) + (c1*g);  v' = (b2*v) + ((c2*g)*g)
 *   w' = w - lr*((m'/bc1) / (sqrt(v'/bc2) + eps) + wd*w)
 * master/exp_avg/exp_avg_sq (fp32[valid_len]) are updated in place, and
 * param_out receives bf16_rne(w') at its base (ZS_OUT_GATHER: param_out +
 * shard_offset; ZS_OUT_SHARD: param_out) followed by +0 in the
 * shard_len - valid_len pad positions.  Nothing beyond valid_len is read or
 * written in the state or gradient buffers, and nothing outside this
 * rank's slot of the gather buffer is written.  bf16_rne: round to nearest
 * even; any NaN becomes the canonical quiet NaN 0x7FC0.
 * Errors: ZS_ENULL, ZS_EINVAL_*, ZS_EALIGN, ZS_EUNSUPPORTED, ZS_ELAUNCH. */
int zero_shard_step(const zs_shard* s, const zs_adamw* h, const uint16_t* const* grad_slices,
                    const float* mean_in, const double* sqnorm, double other_sqnorm,
                    float* master, float* exp_avg, float* exp_avg_sq, uint16_t* param_out,
                    void* stream);

/* Cast and pack only: param_out (placed as in zero_shard_step) receives
 * bf16_rne(master[i]) for i < valid_len and +0 in the pads.  "Data
 * parallelism, ZeRO and FSDP", section 2 table (the all-gather of the new
 * weights after the update) and section 3 Theorem (bf16 weights of 2 bytes
 * next to the fp32 master copy); the slot layout of zs_layout.  The step of
 * the all-gather that needs no optimizer work (e.g. to publish weights after
 * loading a checkpoint).  Errors: ZS_ENULL, ZS_EINVAL_*, ZS_EALIGN,
 * ZS_ELAUNCH. */
int shard_pack_gather(const zs_shard* s, const float* master, uint16_t* param_out,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the clip
 * pass of shard_grad_sqnorm with the same arguments except the workspace,
 * computed by the same kernels into the same results bit for bit.  Its
 * block partials live in a static device array of ZS_SCRATCH_BYTES (16 MiB)
 * per device, held from the first use until the process ends; the call
 * itself allocates nothing and needs no zeroed memory.  Every call on one
 * device shares that device's array, so calls that overlap on one device
 * (several streams or host threads at once) race and give wrong results;
 * serialize them.  The array's device address is taken once per device by
 * zs_init or by the first call on that device (outside a capture, see the
 * HIP graph convention above).
 * Errors: as shard_grad_sqnorm without ZS_EWORKSPACE, plus ZS_ESCRATCH when
 * zs_workspace_bytes(s) > ZS_SCRATCH_BYTES (valid_len above
 * 2,146,959,360); nothing is enqueued then. */
int shard_grad_sqnorm_noalloc(const zs_shard* s, const uint16_t* const* grad_slices,
                              float* mean_out, double* sqnorm_out, int32_t accumulate,
                              void* stream);

/* Per-device set-up for the current HIP device: queries its LDS size, raises
 * the kernels' dynamic-LDS limits and takes the address of the static
 * scratch array.  Optional; every entry point does what it needs itself on
 * its first call on a device.  Call it on each device before capturing
 * library calls into a HIP graph.  Returns ZS_OK or ZS_ELAUNCH. */
int zs_init(void);

/* Static description of an error code ("unknown error" otherwise). */
const char* zs_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif
