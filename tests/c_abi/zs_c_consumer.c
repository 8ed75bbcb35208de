/*
 * A plain C program that uses libzero_shard.so through include/zero_shard.h
 * only (no Python, no torch): the C ABI as a C caller sees it.
 *
 *   zs_c_consumer host   layout, accounting, errors and strings; no GPU.
 *   zs_c_consumer gpu    one clipped optimizer step of a small ragged shard
 *                        on device 0 (hipMalloc'd buffers, the null
 *                        stream), checked bit for bit against the CPU
 *                        oracle (oracle/zs_oracle.h, test code only).
 *
 * Prints one line per check and exits 0 only if every check passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero_shard.h"
#include "zs_oracle.h"

static int failures = 0;

#define CHECK(cond, ...)                                                        \
    do {                                                                        \
        if (cond) {                                                             \
            printf("ok   ");                                                    \
        } else {                                                                \
            printf("FAIL ");                                                    \
            ++failures;                                                         \
        }                                                                       \
        printf(__VA_ARGS__);                                                    \
        printf("\n");                                                           \
    } while (0)

static int host_checks(void)
{
    zs_shard s;
    /* the GPT-2-small shard of rank 3 (S a multiple of 8 * 128) */
    CHECK(zs_layout(124439808, 8, 3, 1024, 2, ZS_OUT_GATHER, &s) == ZS_OK, "zs_layout ok");
    CHECK(s.shard_len == 15555584 && s.shard_offset == 46666752 && s.valid_len == 15555584,
          "gpt2_small rank 3: S %lld, offset %lld, V %lld", (long long)s.shard_len,
          (long long)s.shard_offset, (long long)s.valid_len);
    CHECK(zs_layout(124439808, 8, 7, 1024, 2, ZS_OUT_GATHER, &s) == ZS_OK &&
              s.valid_len == 15550720,
          "gpt2_small rank 7: V %lld (4,864 pads)", (long long)s.valid_len);
    CHECK(zs_layout(0, 8, 0, 1, 2, ZS_OUT_GATHER, &s) == ZS_EINVAL_PSI, "psi 0 rejected");
    CHECK(zs_layout(10, 0, 0, 1, 2, ZS_OUT_GATHER, &s) == ZS_EINVAL_ND, "n_d 0 rejected");
    CHECK(zs_layout(10, 4, 4, 1, 2, ZS_OUT_GATHER, &s) == ZS_EINVAL_RANK, "rank 4 of 4 rejected");
    CHECK(zs_layout(10, 4, 0, 1, 9, ZS_OUT_GATHER, &s) == ZS_EINVAL_STAGE, "stage 9 rejected");
    /* the Theorem's table for 7B over 8 ranks: 112, 38.5, 26.25, 14 GB */
    CHECK(fabs(zs_state_bytes(7e9, 8, 0, 12.0) - 112e9) < 1 &&
              fabs(zs_state_bytes(7e9, 8, 1, 12.0) - 38.5e9) < 1 &&
              fabs(zs_state_bytes(7e9, 8, 2, 12.0) - 26.25e9) < 1 &&
              fabs(zs_state_bytes(7e9, 8, 3, 12.0) - 14e9) < 1,
          "state bytes 7B / 8 ranks");
    CHECK(zs_state_bytes(-1, 8, 0, 12.0) < 0, "negative psi -> -1");
    CHECK(zs_layout(7000000000LL, 8, 3, 1, 2, ZS_OUT_GATHER, &s) == ZS_OK &&
              zs_workspace_bytes(&s) >= 8 * (875000000 / 4096),
          "workspace for 875M parameters: %zu bytes", zs_workspace_bytes(&s));
    CHECK(strcmp(zs_strerror(ZS_OK), "ok") == 0 && strcmp(zs_strerror(-999), "unknown error") == 0,
          "zs_strerror");
    /* argument errors are reported before anything is touched */
    zs_layout(1000, 4, 1, 8, 2, ZS_OUT_GATHER, &s);
    zs_adamw h = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1, 0.0};
    CHECK(zero_shard_step(&s, &h, NULL, NULL, NULL, 0.0, NULL, NULL, NULL, NULL, NULL) ==
              ZS_ENULL,
          "step without a gradient source -> ZS_ENULL");
    h.beta1 = 1.0;
    float dummy[8];
    CHECK(zero_shard_step(&s, &h, NULL, dummy, NULL, 0.0, dummy, dummy, dummy, NULL, NULL) ==
              ZS_EINVAL_HPARAM,
          "beta1 = 1 -> ZS_EINVAL_HPARAM");
    zs_reduce r = {ZS_GRAD_BF16, 0, 1, 0, NULL};
    int64_t zero_tokens[4] = {0, 0, 0, 0};
    const void* fake[4] = {dummy, dummy, dummy, dummy};
    r.rank_tokens = zero_tokens;
    CHECK(shard_grad_reduce(&s, &r, fake, dummy, NULL, 0, NULL, 0, NULL) == ZS_EZERO_TOKENS,
          "zero global token count -> ZS_EZERO_TOKENS");
    return failures;
}

/* xorshift64* for the test's inputs (not part of the method) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normalish(double sigma)   /* sum of 4 uniforms, centred: fine for a test */
{
    double x = uniform01() + uniform01() + uniform01() + uniform01() - 2.0;
    return (float)(x * sigma * 1.7320508);
}

#define HIPCHECK(call)                                                          \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));              \
            return 1;                                                           \
        }                                                                       \
    } while (0)

static int gpu_checks(void)
{
    const int64_t psi = 100003;
    const int32_t n_d = 4, rank = 3;
    zs_shard s;
    if (zs_layout(psi, n_d, rank, 8, 2, ZS_OUT_GATHER, &s) != ZS_OK) return 1;
    const int64_t S = s.shard_len, V = s.valid_len, off = s.shard_offset;
    printf("shard: S %lld, V %lld (%lld pads), offset %lld\n", (long long)S, (long long)V,
           (long long)(S - V), (long long)off);

    uint16_t* h_sl = malloc(sizeof(uint16_t) * (size_t)(n_d * S));
    float* h_w = malloc(sizeof(float) * (size_t)V);
    float* h_m = malloc(sizeof(float) * (size_t)V);
    float* h_v = malloc(sizeof(float) * (size_t)V);
    for (int64_t i = 0; i < n_d * S; ++i) h_sl[i] = 0x7F80;   /* +Inf junk past V */
    for (int32_t r = 0; r < n_d; ++r)
        for (int64_t i = 0; i < V; ++i) h_sl[r * S + i] = or_bf16_rne(normalish(1e-2));
    for (int64_t i = 0; i < V; ++i) {
        h_w[i] = normalish(0.02);
        h_m[i] = normalish(1e-4);
        h_v[i] = fabsf(normalish(1e-6));
    }

    uint16_t *d_sl, *d_out;
    float *d_w, *d_m, *d_v, *d_mean;
    double *d_q;
    void* d_ws;
    const size_t wsb = zs_workspace_bytes(&s);
    HIPCHECK(hipMalloc((void**)&d_sl, sizeof(uint16_t) * (size_t)(n_d * S)));
    HIPCHECK(hipMalloc((void**)&d_out, sizeof(uint16_t) * (size_t)(n_d * S)));
    HIPCHECK(hipMalloc((void**)&d_w, sizeof(float) * (size_t)V));
    HIPCHECK(hipMalloc((void**)&d_m, sizeof(float) * (size_t)V));
    HIPCHECK(hipMalloc((void**)&d_v, sizeof(float) * (size_t)V));
    HIPCHECK(hipMalloc((void**)&d_mean, sizeof(float) * (size_t)V));
    HIPCHECK(hipMalloc((void**)&d_q, sizeof(double)));
    HIPCHECK(hipMalloc(&d_ws, wsb));
    HIPCHECK(hipMemcpy(d_sl, h_sl, sizeof(uint16_t) * (size_t)(n_d * S), hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_w, h_w, sizeof(float) * (size_t)V, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_m, h_m, sizeof(float) * (size_t)V, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_v, h_v, sizeof(float) * (size_t)V, hipMemcpyHostToDevice));
    uint16_t* h_out = malloc(sizeof(uint16_t) * (size_t)(n_d * S));
    for (int64_t i = 0; i < n_d * S; ++i) h_out[i] = 0x7FC1;   /* sentinel */
    HIPCHECK(hipMemcpy(d_out, h_out, sizeof(uint16_t) * (size_t)(n_d * S), hipMemcpyHostToDevice));

    const uint16_t* slices[4];
    for (int32_t r = 0; r < n_d; ++r) slices[r] = d_sl + r * S;
    zs_adamw h = {3e-4, 0.9, 0.999, 1e-8, 0.1, 7, 0.05};
    int rc = shard_grad_sqnorm(&s, slices, d_mean, d_ws, wsb, d_q, 0, NULL);
    CHECK(rc == ZS_OK, "shard_grad_sqnorm: %s", zs_strerror(rc));
    rc = zero_shard_step(&s, &h, NULL, d_mean, d_q, 0.0, d_w, d_m, d_v, d_out, NULL);
    CHECK(rc == ZS_OK, "zero_shard_step: %s", zs_strerror(rc));
    HIPCHECK(hipDeviceSynchronize());

    float* g_w = malloc(sizeof(float) * (size_t)V);
    float* g_m = malloc(sizeof(float) * (size_t)V);
    float* g_v = malloc(sizeof(float) * (size_t)V);
    double g_q = 0.0;
    HIPCHECK(hipMemcpy(g_w, d_w, sizeof(float) * (size_t)V, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(g_m, d_m, sizeof(float) * (size_t)V, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(g_v, d_v, sizeof(float) * (size_t)V, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(&g_q, d_q, sizeof(double), hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(h_out, d_out, sizeof(uint16_t) * (size_t)(n_d * S), hipMemcpyDeviceToHost));

    /* the oracle on the same inputs */
    or_hparams oh = {h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.step, h.max_grad_norm};
    const uint16_t* osl[4];
    for (int32_t r = 0; r < n_d; ++r) osl[r] = h_sl + r * S;
    uint16_t* o_out = malloc(sizeof(uint16_t) * (size_t)S);
    double o_q = 0.0;
    float o_coef = 0.0f;
    rc = or_shard_step(n_d, S, V, &oh, osl, 0.0, h_w, h_m, h_v, o_out, &o_q, &o_coef);
    CHECK(rc == 0, "oracle step");
    CHECK(o_coef < 1.0f, "the clip is active (coef %.6f)", (double)o_coef);
    CHECK(fabs(g_q - o_q) <= 1e-12 * o_q, "squared norm %.17g vs oracle %.17g", g_q, o_q);
    CHECK(memcmp(g_w, h_w, sizeof(float) * (size_t)V) == 0, "master weights bit-exact");
    CHECK(memcmp(g_m, h_m, sizeof(float) * (size_t)V) == 0, "exp_avg bit-exact");
    CHECK(memcmp(g_v, h_v, sizeof(float) * (size_t)V) == 0, "exp_avg_sq bit-exact");
    CHECK(memcmp(h_out + off, o_out, sizeof(uint16_t) * (size_t)S) == 0,
          "bf16 slot (values and pads) bit-exact");
    int outside_ok = 1;
    for (int64_t i = 0; i < n_d * S; ++i)
        if ((i < off || i >= off + S) && h_out[i] != 0x7FC1) outside_ok = 0;
    CHECK(outside_ok, "other ranks' slots untouched");

    hipFree(d_sl); hipFree(d_out); hipFree(d_w); hipFree(d_m); hipFree(d_v);
    hipFree(d_mean); hipFree(d_q); hipFree(d_ws);
    free(h_sl); free(h_w); free(h_m); free(h_v); free(h_out); free(g_w); free(g_m); free(g_v);
    free(o_out);
    return failures;
}

int main(int argc, char** argv)
{
    if (argc < 2 || (strcmp(argv[1], "host") != 0 && strcmp(argv[1], "gpu") != 0)) {
        fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
        return 2;
    }
    const int bad = strcmp(argv[1], "host") == 0 ? host_checks() : gpu_checks();
    printf("%s: %d failure(s)\n", argv[1], bad);
    return bad == 0 ? 0 : 1;
}
