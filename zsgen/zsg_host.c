/*
 * zsg_host.c -- host side of the seeded input generator (definition in
 * zsg_def.h).  Multithreaded with pthreads: the range is split into
 * contiguous pieces, one per thread; the values do not depend on the split.
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -pthread.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ZSG_FN static inline
#include "zsg_def.h"

#define ZSG_HOST_FSQRT(x) sqrtf(x)

typedef struct {
    int kind;                 /* 0: f32 normal, 1: bf16 normal, 2: f32 gather, 3: bf16 gather */
    uint64_t key, key_mask, key_val;
    double sigma, p_out, sigma_out;
    int absval;
    int64_t start, n;         /* fill: elements start .. start+n-1 */
    const int64_t* idx;       /* gather: element indices */
    void* out;
} job_t;

static double normal_at(uint64_t key, int64_t i)
{
    double z0, z1;
    ZSG_NORMAL_PAIR(key, (uint64_t)i >> 1, z0, z1, ZSG_HOST_FSQRT);
    return (i & 1) ? z1 : z0;
}

static double value_at(const job_t* jb, int64_t i, double z)
{
    double x = z * jb->sigma;
    if (jb->p_out > 0.0) {
        uint64_t h = zsg_draw(jb->key_mask, (uint64_t)i);
        double u = (double)(h >> 11) * (1.0 / 9007199254740992.0);
        if (u < jb->p_out) x = normal_at(jb->key_val, i) * jb->sigma_out;
    }
    if (jb->absval && x < 0.0) x = -x;
    return x;
}

static void store(const job_t* jb, int64_t pos, double x)
{
    if (jb->kind == 0 || jb->kind == 2) {
        uint32_t b = zsg_trunc_f32(x);
        ((uint32_t*)jb->out)[pos] = b;
    } else {
        ((uint16_t*)jb->out)[pos] = zsg_trunc_bf16(x);
    }
}

static void* run_job(void* p)
{
    const job_t* jb = (const job_t*)p;
    if (jb->kind <= 1) {
        int64_t i = jb->start, end = jb->start + jb->n;
        while (i < end) {
            double z0, z1;
            uint64_t j = (uint64_t)i >> 1;
            ZSG_NORMAL_PAIR(jb->key, j, z0, z1, ZSG_HOST_FSQRT);
            int64_t e0 = (int64_t)(2 * j), e1 = e0 + 1;
            if (e0 >= i && e0 < end) store(jb, e0 - jb->start, value_at(jb, e0, z0));
            if (e1 >= i && e1 < end) store(jb, e1 - jb->start, value_at(jb, e1, z1));
            i = e1 + 1;
        }
    } else {
        for (int64_t k = 0; k < jb->n; ++k) {
            int64_t i = jb->idx[k];
            store(jb, k, value_at(jb, i, normal_at(jb->key, i)));
        }
    }
    return NULL;
}

static int run(job_t base, int nthreads, int64_t total)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (total < 4096 * (int64_t)nthreads) nthreads = 1;
    job_t jobs[256];
    pthread_t th[256];
    int64_t per = (total + nthreads - 1) / nthreads;
    per = (per + 1) & ~(int64_t)1;
    int used = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t a = (int64_t)t * per, b = a + per;
        if (a >= total) break;
        if (b > total) b = total;
        jobs[t] = base;
        if (base.kind <= 1) {
            jobs[t].start = base.start + a;
            jobs[t].n = b - a;
            size_t esz = base.kind == 0 ? 4 : 2;
            jobs[t].out = (char*)base.out + (size_t)a * esz;
        } else {
            jobs[t].idx = base.idx + a;
            jobs[t].n = b - a;
            size_t esz = base.kind == 2 ? 4 : 2;
            jobs[t].out = (char*)base.out + (size_t)a * esz;
        }
        used = t + 1;
    }
    for (int t = 1; t < used; ++t)
        if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) return -1;
    if (used > 0) run_job(&jobs[0]);
    for (int t = 1; t < used; ++t) pthread_join(th[t], NULL);
    return 0;
}

static job_t make_job(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
                      double sigma, int absval, double p_out, double sigma_out)
{
    job_t jb;
    jb.kind = 0;
    jb.key = zsg_key(seed, stream, rank, step);
    jb.key_mask = zsg_key(seed, stream | ZSG_SUBSTREAM_MASK, rank, step);
    jb.key_val = zsg_key(seed, stream | ZSG_SUBSTREAM_OUTLIER, rank, step);
    jb.sigma = sigma;
    jb.p_out = p_out;
    jb.sigma_out = sigma_out;
    jb.absval = absval;
    jb.start = 0;
    jb.n = 0;
    jb.idx = NULL;
    jb.out = NULL;
    return jb;
}

/* fp32 values sigma * N(0,1) (|.| if absval) at elements start .. start+n-1. */
int zsg_fill_f32(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
                 double sigma, int absval, int64_t start, int64_t n, float* out,
                 int nthreads)
{
    if (n <= 0) return 0;
    if (start < 0 || !out) return -1;
    job_t jb = make_job(seed, stream, rank, step, sigma, absval, 0.0, 0.0);
    jb.kind = 0;
    jb.start = start;
    jb.n = n;
    jb.out = out;
    return run(jb, nthreads, n);
}

/* bf16 values sigma * N(0,1); with probability p_out an element is replaced
 * by sigma_out * N(0,1) from an independent stream. */
int zsg_fill_bf16(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
                  double sigma, double p_out, double sigma_out, int64_t start,
                  int64_t n, uint16_t* out, int nthreads)
{
    if (n <= 0) return 0;
    if (start < 0 || !out) return -1;
    job_t jb = make_job(seed, stream, rank, step, sigma, 0, p_out, sigma_out);
    jb.kind = 1;
    jb.start = start;
    jb.n = n;
    jb.out = out;
    return run(jb, nthreads, n);
}

int zsg_gather_f32(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
                   double sigma, int absval, const int64_t* idx, int64_t n,
                   float* out, int nthreads)
{
    if (n <= 0) return 0;
    if (!idx || !out) return -1;
    job_t jb = make_job(seed, stream, rank, step, sigma, absval, 0.0, 0.0);
    jb.kind = 2;
    jb.idx = idx;
    jb.n = n;
    jb.out = out;
    return run(jb, nthreads, n);
}

int zsg_gather_bf16(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step,
                    double sigma, double p_out, double sigma_out, const int64_t* idx,
                    int64_t n, uint16_t* out, int nthreads)
{
    if (n <= 0) return 0;
    if (!idx || !out) return -1;
    job_t jb = make_job(seed, stream, rank, step, sigma, 0, p_out, sigma_out);
    jb.kind = 3;
    jb.idx = idx;
    jb.n = n;
    jb.out = out;
    return run(jb, nthreads, n);
}
