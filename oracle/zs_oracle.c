/*
 * zs_oracle.c -- CPU oracle of the sharded AdamW step (test infrastructure
 * only; see zs_oracle.h for the citation keys and the floating-point
 * contract).  Single-threaded and deliberately plain: every loop walks its
 * elements in ascending order and every expression is written in the order
 * the pages write it.  Build: gcc -O2 -ffp-contract=off -fno-fast-math.
 */
#include "zs_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- layout --------------------------------------------------------------- */

int or_layout(int64_t psi, int32_t n_d, int32_t rank, int64_t align,
              int32_t stage, int64_t* shard_len, int64_t* shard_offset,
              int64_t* valid_len)
{
    if (psi <= 0) return -1;
    if (n_d < 1) return -2;
    if (rank < 0 || rank >= n_d) return -3;
    if (align < 1) return -4;
    if (stage < 0 || stage > 3) return -5;

    int64_t S, off, V;
    if (stage == 0) {
        /* DDP: nothing is sharded, the whole vector is this rank's. */
        S = ((psi + align - 1) / align) * align;
        off = 0;
        V = psi;
    } else {
        int64_t chunk = (psi + n_d - 1) / n_d;          /* ceil(psi / n_d)  */
        S = ((chunk + align - 1) / align) * align;      /* round up to align */
        off = (int64_t)rank * S;
        V = psi - off;
        if (V < 0) V = 0;
        if (V > S) V = S;
    }
    *shard_len = S;
    *shard_offset = off;
    *valid_len = V;
    return 0;
}

/* ---- accounting ----------------------------------------------------------- */

double or_state_bytes(double psi, int32_t n_d, int32_t stage, double K)
{
    switch (stage) {
    case 0: return (4.0 + K) * psi;
    case 1: return 4.0 * psi + K * psi / n_d;
    case 2: return 2.0 * psi + (2.0 + K) * psi / n_d;
    case 3: return (4.0 + K) * psi / n_d;
    default: return -1.0;
    }
}

double or_comm_elems(double psi, int32_t stage)
{
    switch (stage) {
    case 0: case 1: case 2: return 2.0 * psi;
    case 3: return 3.0 * psi;
    default: return -1.0;
    }
}

double or_comm_bytes(double psi, int32_t n_d, int32_t stage,
                     double bytes_per_elem)
{
    double e = or_comm_elems(psi, stage);
    if (e < 0) return -1.0;
    return e * bytes_per_elem * (double)(n_d - 1) / (double)n_d;
}

double or_comm_elems_accum(double psi, int32_t stage, int32_t m)
{
    switch (stage) {
    case 0: case 1: return 2.0 * psi;
    case 2: return m * psi + psi;
    case 3: return 3.0 * m * psi;
    default: return -1.0;
    }
}

double or_hsdp_state_bytes(double psi, int32_t g, double K)
{
    return (4.0 + K) * psi / g;
}

double or_hsdp_intra_bytes(double psi, int32_t g, double bytes_per_elem)
{
    return 3.0 * bytes_per_elem * psi * (double)(g - 1) / (double)g;
}

double or_hsdp_inter_bytes(double psi, int32_t n_d, int32_t g,
                           double bytes_per_elem)
{
    double r = (double)n_d / (double)g;
    double shard = bytes_per_elem * psi / g;
    return 2.0 * (r - 1.0) / r * shard;
}

/* ---- bfloat16 ------------------------------------------------------------- */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

uint16_t or_bf16_rne(float x)
{
    uint32_t u = f32_bits(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)0x7FC0u;   /* any NaN: the canonical quiet NaN */
    uint32_t hi = u >> 16;          /* kept: sign, exponent, 7 mantissa bits */
    uint32_t lo = u & 0xFFFFu;      /* dropped bits */
    /* Nearest; on an exact tie pick the even kept value.  A carry out of the
     * mantissa moves to the next binade (or to Inf), which is the correct
     * rounded result. */
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

float or_bf16_to_f32(uint16_t h)
{
    return bits_f32((uint32_t)h << 16);
}

void or_bf16_rne_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_rne(x[i]);
}

/* ---- O1 ---------------------------------------------------------------- */

void or_reduce_mean(int32_t n_d, const uint16_t* const* slices, int64_t n,
                    float* g_out)
{
    const float nd = (float)n_d;
    for (int64_t i = 0; i < n; ++i) {
        float s = or_bf16_to_f32(slices[0][i]);
        for (int32_t r = 1; r < n_d; ++r)
            s = s + or_bf16_to_f32(slices[r][i]);
        g_out[i] = s / nd;
    }
}

void or_reduce_mean_f32in(int32_t n_d, const float* const* slices, int64_t n,
                          float* g_out)
{
    const float ranks = (float)n_d;
    for (int64_t i = 0; i < n; ++i) {
        float sum = slices[0][i];
        for (int32_t r = 1; r < n_d; ++r)
            sum = sum + slices[r][i];
        g_out[i] = sum / ranks;
    }
}

int or_token_weights(int32_t n_d, const int64_t* tokens, float* w_out)
{
    double T = 0.0;
    for (int32_t r = 0; r < n_d; ++r) {
        if (tokens[r] < 0) return -1;
        T += (double)tokens[r];
    }
    if (T == 0.0) return -2;
    for (int32_t r = 0; r < n_d; ++r) w_out[r] = (float)((double)tokens[r] / T);
    return 0;
}

static float slice_value(int32_t f32in, const void* slice, int64_t i)
{
    if (f32in) return ((const float*)slice)[i];
    return or_bf16_to_f32(((const uint16_t*)slice)[i]);
}

void or_reduce_weighted(int32_t n_d, int32_t f32in, const void* const* slices,
                        const float* w, int64_t n, float* g_out)
{
    for (int64_t i = 0; i < n; ++i) {
        float s = w[0] * slice_value(f32in, slices[0], i);
        for (int32_t r = 1; r < n_d; ++r) {
            const float p = w[r] * slice_value(f32in, slices[r], i);
            s = s + p;
        }
        g_out[i] = s;
    }
}

void or_accumulate(int64_t n, const float* r_j, int32_t j, int32_t m,
                   float* acc)
{
    const float mf = (float)m;
    for (int64_t i = 0; i < n; ++i) {
        float a = (j == 0) ? r_j[i] : acc[i] + r_j[i];
        if (j == m - 1 && m > 1) a = a / mf;
        acc[i] = a;
    }
}

/* ---- O2 / O3 -------------------------------------------------------------- */

void or_sqacc_init(or_sqacc* a)
{
    memset(a, 0, sizeof(*a));
}

int64_t or_sqacc_size(void) { return (int64_t)sizeof(or_sqacc); }

void or_sqacc_add(or_sqacc* a, const float* g, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = f32_bits(g[i]);
        uint32_t e = (u >> 23) & 0xFFu;
        uint32_t frac = u & 0x7FFFFFu;
        if (e == 0xFFu) {                       /* Inf or NaN */
            if (frac) a->has_nan = 1; else a->has_inf = 1;
            continue;
        }
        /* |g| = M * 2^(max(e,1) - 150), M < 2^24; g^2 = M^2 * 2^(2(max(e,1) - 150)) */
        uint64_t M = (e == 0) ? frac : (frac | 0x800000u);
        uint64_t sq = M * M;                     /* < 2^48, exact */
        uint32_t b = (e == 0) ? 1u : e;
        uint64_t before = a->lo[b];
        a->lo[b] = before + sq;
        if (a->lo[b] < before) a->hi[b] += 1u;  /* carry */
    }
}

/* Big integer of 32-bit limbs, in units of 2^-298 (the weight of bucket 1). */
#define OR_LIMBS 24

static void big_add_shifted(uint32_t* L, uint64_t lo, uint64_t hi, int shift)
{
    /* add (hi:lo) * 2^shift into L, one bit at a time (slow, plain) */
    for (int bit = 0; bit < 128; ++bit) {
        uint64_t word = bit < 64 ? lo : hi;
        if (!((word >> (bit & 63)) & 1u)) continue;
        int pos = shift + bit;
        int limb = pos / 32, off = pos % 32;
        uint64_t carry = (uint64_t)1 << off;
        while (carry && limb < OR_LIMBS) {
            uint64_t s = (uint64_t)L[limb] + carry;
            L[limb] = (uint32_t)s;
            carry = s >> 32;
            ++limb;
        }
    }
}

static int big_bit(const uint32_t* L, int i)
{
    return (int)((L[i / 32] >> (i % 32)) & 1u);
}

double or_sqacc_value(const or_sqacc* a)
{
    if (a->has_nan) return NAN;
    if (a->has_inf) return INFINITY;
    uint32_t L[OR_LIMBS];
    memset(L, 0, sizeof(L));
    for (int b = 1; b < 255; ++b)
        if (a->lo[b] || a->hi[b]) big_add_shifted(L, a->lo[b], a->hi[b], 2 * (b - 1));
    int top = -1;
    for (int i = OR_LIMBS * 32 - 1; i >= 0; --i)
        if (big_bit(L, i)) { top = i; break; }
    if (top < 0) return 0.0;
    if (top < 53) {                             /* fits 53 bits: exact */
        uint64_t v = 0;
        for (int i = top; i >= 0; --i) v = (v << 1) | (uint64_t)big_bit(L, i);
        return ldexp((double)v, -298);
    }
    uint64_t mant = 0;                          /* bits top .. top-52 */
    for (int i = top; i >= top - 52; --i) mant = (mant << 1) | (uint64_t)big_bit(L, i);
    int round = big_bit(L, top - 53);
    int sticky = 0;
    for (int i = top - 54; i >= 0 && !sticky; --i) sticky = big_bit(L, i);
    if (round && (sticky || (mant & 1u))) {
        mant += 1;
        if (mant == ((uint64_t)1 << 53)) { mant >>= 1; top += 1; }
    }
    return ldexp((double)mant, top - 52 - 298);
}

double or_sqnorm(const float* g, int64_t n)
{
    or_sqacc a;
    or_sqacc_init(&a);
    or_sqacc_add(&a, g, n);
    return or_sqacc_value(&a);
}

float or_clip_coef(double Q, double max_norm)
{
    double c = max_norm / (sqrt(Q) + 1e-6);
    if (c > 1.0) c = 1.0;           /* NaN fails the test and stays NaN */
    return (float)c;
}

/* ---- O4 ------------------------------------------------------------------- */

void or_make_consts(const or_hparams* h, or_consts* c)
{
    double t = (double)h->step;
    c->b1 = (float)h->beta1;
    c->b2 = (float)h->beta2;
    c->c1 = (float)(1.0 - h->beta1);
    c->c2 = (float)(1.0 - h->beta2);
    c->bc1 = (float)(1.0 - pow(h->beta1, t));
    c->bc2 = (float)(1.0 - pow(h->beta2, t));
    c->lr = (float)h->lr;
    c->wd = (float)h->weight_decay;
    c->eps = (float)h->eps;
}

void or_adamw_f32(const or_consts* c, int64_t n, const float* g,
                  int use_coef, float coef, float* w, float* m, float* v)
{
    for (int64_t i = 0; i < n; ++i) {
        float gi = g[i];
        if (use_coef) gi = gi * coef;
        float mi = (c->b1 * m[i]) + (c->c1 * gi);
        float vi = (c->b2 * v[i]) + ((c->c2 * gi) * gi);
        float mh = mi / c->bc1;
        float vh = vi / c->bc2;
        float u = (mh / (sqrtf(vh) + c->eps)) + (c->wd * w[i]);
        w[i] = w[i] - (c->lr * u);
        m[i] = mi;
        v[i] = vi;
    }
}

/* ---- O5 ------------------------------------------------------------------- */

void or_pack(int64_t shard_len, int64_t valid_len, const float* w,
             uint16_t* out)
{
    for (int64_t i = 0; i < valid_len; ++i) out[i] = or_bf16_rne(w[i]);
    for (int64_t i = valid_len; i < shard_len; ++i) out[i] = 0;
}

/* ---- whole shard step ------------------------------------------------------ */

int or_shard_step(int32_t n_d, int64_t shard_len, int64_t valid_len,
                  const or_hparams* h, const uint16_t* const* slices,
                  double other_sqnorm, float* w, float* m, float* v,
                  uint16_t* out, double* local_sqnorm_out, float* coef_out)
{
    float* g = NULL;
    if (valid_len > 0) {
        g = (float*)malloc((size_t)valid_len * sizeof(float));
        if (!g) return -1;
        or_reduce_mean(n_d, slices, valid_len, g);
    }
    int clip = h->max_grad_norm > 0.0;
    double q = or_sqnorm(g, valid_len);
    float coef = 1.0f;
    if (clip) coef = or_clip_coef(q + other_sqnorm, h->max_grad_norm);
    or_consts c;
    or_make_consts(h, &c);
    if (valid_len > 0) or_adamw_f32(&c, valid_len, g, clip, coef, w, m, v);
    or_pack(shard_len, valid_len, w, out);
    if (local_sqnorm_out) *local_sqnorm_out = q;
    if (coef_out) *coef_out = coef;
    free(g);
    return 0;
}

/* ---- fp64 mode ------------------------------------------------------------- */

void or_reduce_mean_f64(int32_t n_d, const double* const* slices, int64_t n,
                        double* g_out)
{
    for (int64_t i = 0; i < n; ++i) {
        double s = slices[0][i];
        for (int32_t r = 1; r < n_d; ++r) s = s + slices[r][i];
        g_out[i] = s / (double)n_d;
    }
}

void or_adamw_f64(const or_hparams* h, int64_t n, const double* g,
                  double* w, double* m, double* v)
{
    double b1 = h->beta1, b2 = h->beta2, t = (double)h->step;
    double bc1 = 1.0 - pow(b1, t), bc2 = 1.0 - pow(b2, t);
    for (int64_t i = 0; i < n; ++i) {
        double mi = b1 * m[i] + (1.0 - b1) * g[i];
        double vi = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
        double mh = mi / bc1, vh = vi / bc2;
        w[i] = w[i] - h->lr * (mh / (sqrt(vh) + h->eps) + h->weight_decay * w[i]);
        m[i] = mi;
        v[i] = vi;
    }
}
