/*
 * zs_oracle.h -- CPU oracle for one GPU's share of the ZeRO / FSDP sharded
 * optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source, header, table or helper with
 * the HIP library; both sides are written separately from the same pages.
 *
 * Plain, slow, single-threaded C.  Every function states the passage of the
 * pages it follows.  The pages are cited by title and section:
 *   [DPZ]  "Data parallelism, ZeRO and FSDP" (ML Systems, Lesson 8,
 *          learn.mohebi.ai)
 *   [DDB]  "Distributed Training Basics -- DDP and FSDP" (dineshblog.com)
 *   [TAI]  "Data parallelism, collectives and ZeRO/FSDP" (techaiinterview.com)
 *   [GUS]  "Distributed Training: FSDP, DeepSpeed, and Megatron"
 *          (thegustafson.com)
 *
 * Floating-point contract of the fp32 functions: IEEE-754 binary32, round to
 * nearest even, one rounding per written operation, no fused multiply-add
 * (built with -ffp-contract=off), subnormals kept.  sqrtf and '/' are the
 * correctly rounded IEEE operations.
 *
 * Parity status: every function below is pinned by a CPU test against values
 * the pages print, closed forms, a library routine (torch.optim.AdamW,
 * torch.nn.utils.clip_grad_norm_, torch's float->bfloat16 cast) or brute force.
 * One reading is unpinned: whether a real ring's reduction order and dtype
 * would give the same bits (the pages print no such result).
 */
#ifndef ZS_ORACLE_H
#define ZS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- shard layout ------------------------------------------------------ */
/* [DPZ] §2 "What is redundant": rank k owns slice k of the parameters.
 * [DPZ] §3 "How FSDP implements ZeRO-3", step 1: FSDP1 flattens a unit into
 * one vector cut into N_d equal chunks.  Reading: the flat vector of psi
 * elements is padded at its tail to n_d*S, S = roundup(ceil(psi/n_d), align);
 * slot k is [k*S, (k+1)*S); valid_len = clamp(psi - k*S, 0, S).
 * stage 0 (DDP, nothing sharded): every rank owns the whole vector, S =
 * roundup(psi, align), offset 0, valid_len = psi.
 * Returns 0, or -1 psi<=0, -2 n_d<1, -3 rank out of range, -4 align<1,
 * -5 stage not in 0..3. */
int or_layout(int64_t psi, int32_t n_d, int32_t rank, int64_t align,
              int32_t stage, int64_t* shard_len, int64_t* shard_offset,
              int64_t* valid_len);

/* ---- accounting -------------------------------------------------------- */
/* [DPZ] §3 Theorem "ZeRO memory and communication", table and proof steps
 * 1-4: model-state bytes per GPU, weights and grads 2 B each, K optimizer
 * bytes per parameter.  stage 0 (4+K)psi; 1: 4psi + K psi/n_d;
 * 2: 2psi + (2+K) psi/n_d; 3: (4+K) psi/n_d.  Negative -> invalid stage. */
double or_state_bytes(double psi, int32_t n_d, int32_t stage, double K);

/* [DPZ] §3 Theorem, table column "elements sent per GPU per step" and proof
 * steps 5-7: 2psi for stages 0-2, 3psi for stage 3.  Bytes are
 * elems * bytes_per_elem * (n_d-1)/n_d (the sentence under the table). */
double or_comm_elems(double psi, int32_t stage);
double or_comm_bytes(double psi, int32_t n_d, int32_t stage,
                     double bytes_per_elem);

/* [DPZ] §3 "Gradient accumulation", table: elements sent per GPU per
 * optimizer step with m micro-batches.  0,1: 2psi; 2: m psi + psi;
 * 3: 3 m psi. */
double or_comm_elems_accum(double psi, int32_t stage, int32_t m);

/* [DPZ] §3 "How FSDP implements ZeRO-3", step 6 (HSDP): shard inside groups
 * of g GPUs, replicate over r = n_d/g.  State (4+K)psi/g.  Per GPU bytes:
 * inside the group 3 * bytes*psi * (g-1)/g (two all-gathers, one
 * reduce-scatter, no reshard exemption); across groups one all-reduce of the
 * gradient shard, 2 * (r-1)/r * bytes*psi/g. */
double or_hsdp_state_bytes(double psi, int32_t g, double K);
double or_hsdp_intra_bytes(double psi, int32_t g, double bytes_per_elem);
double or_hsdp_inter_bytes(double psi, int32_t n_d, int32_t g,
                           double bytes_per_elem);

/* ---- bfloat16 ------------------------------------------------------------ */
/* [DPZ] §3 Notation: weights and gradients are bf16.  Reading: float->bf16 is
 * round to nearest, ties to even on the 16 dropped bits; +-Inf, +-0 kept;
 * overflow rounds to Inf; any NaN becomes the canonical quiet NaN 0x7FC0
 * (IEEE 754 leaves the sign and payload of an arithmetic NaN open, so only
 * a canonical NaN makes the packed bits well defined). */
uint16_t or_bf16_rne(float x);
float    or_bf16_to_f32(uint16_t h);   /* exact widening */
void     or_bf16_rne_array(const float* x, int64_t n, uint16_t* out);

/* ---- O1: the reduce-scatter's local reduction ---------------------------- */
/* [DPZ] §2 "Two GPUs, one batch" and Proposition "DDP is exact", step 3: the
 * rank gradients are averaged.  [DPZ] remark after that proof: the order of
 * the sum changes the last bits.  Reading: widen each rank's bf16 value
 * exactly to fp32, add in rank order 0,1,...,n_d-1 starting from rank 0's
 * value, then divide by (float)n_d once (correctly rounded).
 * slices[r][i] is element i of rank r's slice, i in [0, n). */
void or_reduce_mean(int32_t n_d, const uint16_t* const* slices, int64_t n,
                    float* g_out);

/* ---- reductions beyond the bf16 mean --------------------------------------- */
/* fp32 gradient slices.  [DPZ] "tokens that hide the all-reduce" (fp32
 * gradient reduction doubles the bytes) and §6 "Where it shows up" (Llama 3
 * reduce-scattered gradients in fp32); [DDB] "FSDP1 and FSDP2: explicitly
 * different versioned paths", its mixed-precision policy
 * reduce_dtype=torch.float32.  Reading: the rank-order fp32 sum of
 * or_reduce_mean, from fp32 inputs, divided by (float)n_d once. */
void or_reduce_mean_f32in(int32_t n_d, const float* const* slices, int64_t n,
                          float* g_out);

/* Token-weighted reduction.  [DPZ] §7 "Common mistakes", the item on sum
 * versus mean and unequal token counts: when the loss is a mean over tokens
 * and the ranks hold different numbers of tokens, the ranks' gradients are
 * combined in proportion to those counts.  [DDB] "DDP: replicated state, partitioned
 * examples": ranks with 2 and 6 tokens and local mean losses 3 and 1 give
 * (2*3+6*1)/8 = 1.5, not 2; a zero-token rank contributes a zero and still
 * takes part; [DDB] "Practice and worked answers", item 4: if the global
 * count is zero every rank rejects the update.
 * Reading: slice r holds the gradient of rank r's local mean loss;
 * w_r = f32(n_r / T), T = sum of n_r, in double; then
 * g = (((w_0*G_0) + (w_1*G_1)) + ...) in rank order, every product and every
 * sum rounded to fp32.  or_token_weights returns 0, -1 if a count is
 * negative, -2 if T == 0 (the update is rejected; w_out untouched).
 * f32in: 0 -> slices are bf16 (uint16_t), 1 -> fp32. */
int  or_token_weights(int32_t n_d, const int64_t* tokens, float* w_out);
void or_reduce_weighted(int32_t n_d, int32_t f32in, const void* const* slices,
                        const float* w, int64_t n, float* g_out);

/* ZeRO-2 gradient accumulation.  [DPZ] §3 "Gradient accumulation": m
 * micro-batches run one after the other and their gradients are added
 * before one optimizer step; ZeRO-2 keeps no full gradient, so it
 * reduce-scatters after every micro-batch (table row ZeRO-2).  [DDB]
 * "Accumulation, clipping and scaling measurements": clipping and the
 * optimizer act at the effective-update boundary, after the last
 * micro-batch.  Reading:
 * micro-batch j's reduced slice r_j (any reduction above) is added in fp32
 * into a persistent shard accumulator in micro-batch order: acc = r_0, then
 * acc = acc + r_j; after the last one (j = m-1) the step's gradient is
 * acc / (float)m, correctly rounded: the mean over the m micro-batches.
 * For m == 1, acc = r_0. */
void or_accumulate(int64_t n, const float* r_j, int32_t j, int32_t m,
                   float* acc);

/* ---- O2/O3: global gradient-norm clip ------------------------------------ */
/* [DPZ] §7 "Common mistakes", last item: with sharded gradients the global
 * norm is an all-reduce of the squared shard norms.  [DDB] reference DDP
 * program: clip_grad_norm_(..., 1.) at the update boundary.
 * The squared norm is the plain definition: the exact sum of g_i^2 over the
 * elements, rounded once to double (round to nearest even).  Each g_i^2 of an
 * fp32 g_i is an integer below 2^48 times a power of two, so the accumulator
 * keeps one 128-bit integer sum per exponent; nothing is rounded until
 * or_sqacc_value.  Any NaN makes the value NaN, else any Inf makes it +Inf. */
typedef struct {
    uint64_t lo[255], hi[255];   /* bucket e: sum of squared significands of
                                    elements with biased exponent e */
    int32_t has_nan, has_inf;
} or_sqacc;
void   or_sqacc_init(or_sqacc* a);
void   or_sqacc_add(or_sqacc* a, const float* g, int64_t n);
double or_sqacc_value(const or_sqacc* a);
int64_t or_sqacc_size(void);
double or_sqnorm(const float* g, int64_t n);   /* init + add + value */
/* coef = f32(min(1, max_norm / (sqrt(Q) + 1e-6))) in double; a NaN quotient
 * stays NaN (the clamp propagates it), Q = +Inf gives 0.  The 1e-6 is the
 * library call's constant, not printed on the pages. */
float  or_clip_coef(double Q, double max_norm);

/* ---- O4: AdamW, fp32 mixed precision ------------------------------------- */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;            /* t >= 1 */
    double max_grad_norm;    /* <= 0: no clip */
} or_hparams;

/* Scalars rounded once from double to float. */
typedef struct { float b1, b2, c1, c2, bc1, bc2, lr, wd, eps; } or_consts;

/* [DPZ] §5 "In code", the simulator's adamw: bias corrections 1 - beta^t with
 * t counted from 1.  b1=f32(beta1) b2=f32(beta2) c1=f32(1-beta1)
 * c2=f32(1-beta2) bc1=f32(1-pow(beta1,t)) bc2=f32(1-pow(beta2,t)),
 * lr, wd, eps rounded to float. */
void or_make_consts(const or_hparams* h, or_consts* c);

/* [DPZ] §5 "In code", adamw, in the expression order it is written:
 *   (clip only)  g  = g * coef
 *   m' = (b1*m) + (c1*g);  v' = (b2*v) + ((c2*g)*g)
 *   mh = m'/bc1;  vh = v'/bc2
 *   w' = w - lr*((mh / (sqrtf(vh) + eps)) + (wd*w))
 * Weight decay applies to every element (a flat shard has no groups).
 * [DPZ] §2 "What is redundant": the update is elementwise, so a slice needs
 * only its own g, m, v and fp32 master w. */
void or_adamw_f32(const or_consts* c, int64_t n, const float* g,
                  int use_coef, float coef, float* w, float* m, float* v);

/* ---- O5: bf16 cast and pack into the all-gather slot ---------------------- */
/* [DPZ] §2 "The communication is already there", table: after the update
 * rank k's new slice k is all-gathered; [TAI] FSDP diagram: the optimizer
 * hands back a new bf16 shard.  out[i] = bf16(w[i]) for i < valid_len,
 * +0 for valid_len <= i < shard_len.  `out` points at the slot base. */
void or_pack(int64_t shard_len, int64_t valid_len, const float* w,
             uint16_t* out);

/* ---- one whole shard step (O1..O5) ---------------------------------------- */
/* Applies O1; if h->max_grad_norm > 0, O2 over the shard (exact), Q = local +
 * other_sqnorm (stand-in for the scalar all-reduce), O3 coef; O4 on the
 * valid_len elements; O5 into out[0 .. shard_len).  Writes the local
 * sqnorm and coef if the pointers are non-NULL (NaN coef reported as 1 when
 * there is no clip).  Returns 0, or -1 on allocation failure. */
int or_shard_step(int32_t n_d, int64_t shard_len, int64_t valid_len,
                  const or_hparams* h, const uint16_t* const* slices,
                  double other_sqnorm, float* w, float* m, float* v,
                  uint16_t* out, double* local_sqnorm_out, float* coef_out);

/* ---- fp64 mode ---------------------------------------------------------- */
/* The simulator's arithmetic of [DPZ] §5 in double: mean over ranks, then
 * adamw with pow() bias corrections.  Used to reproduce that simulator's
 * sharded-equals-unsharded check. */
void or_reduce_mean_f64(int32_t n_d, const double* const* slices, int64_t n,
                        double* g_out);
void or_adamw_f64(const or_hparams* h, int64_t n, const double* g,
                  double* w, double* m, double* v);

#ifdef __cplusplus
}
#endif
#endif
