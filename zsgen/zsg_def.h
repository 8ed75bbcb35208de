/*
 * zsg_def.h -- definition of the seeded synthetic-input generator.
 *
 * This generator produces the inputs of the sharded optimizer step (master
 * weights, moments, per-rank bf16 gradients) for the tests and the
 * benchmark.  It holds none of the optimizer step's arithmetic.  The same
 * definition is compiled for the host (zsg_host.c, used by the CPU oracle's
 * side) and for the GPU (zsg_device.hip, which fills HBM directly); every
 * operation is an integer operation or an IEEE-754 double +, -, *, / (each
 * correctly rounded on both), so both produce the same bits.  The includer
 * defines ZSG_FN (the function qualifier) before including this file.
 *
 * Definition.
 *  - mix64: the SplitMix64 output function (Steele, Lea and Flood,
 *    "Fast splittable pseudorandom number generators", OOPSLA 2014; the
 *    constants of Vigna's public splitmix64.c).
 *  - A stream key is derived from (seed, stream id, rank, step); the c-th
 *    draw of a stream is mix64(key + c * 0x9E3779B97F4A7C15).
 *  - Standard normals: Marsaglia and Bray's polar method ("A convenient
 *    method for generating normal variables", SIAM Review 6, 1964).  Pair j
 *    takes draws 64j, 64j+1, ... until one lands inside the unit disc; both
 *    coordinates become normals (element 2j and 2j+1).  The natural log is
 *    the atanh series of (m-1)/(m+1) after exponent extraction, and the
 *    square root is two Newton steps from a float seed, so no libm routine
 *    whose last bit could differ between host and device is involved.
 *  - Quantisation to fp32 or bf16 is truncation of the double toward zero
 *    (the generator's own rule; magnitudes below the smallest normal become
 *    signed zero).
 */
#ifndef ZSG_DEF_H
#define ZSG_DEF_H

#include <stdint.h>

#define ZSG_GOLDEN 0x9E3779B97F4A7C15ull

ZSG_FN uint64_t zsg_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* stream < 2^16, rank < 2^16, step < 2^32 */
ZSG_FN uint64_t zsg_key(uint64_t seed, uint32_t stream, uint32_t rank, uint32_t step)
{
    uint64_t k = zsg_mix64(seed * ZSG_GOLDEN + 0x632BE59BD9B4E019ull);
    return zsg_mix64(k ^ ((uint64_t)stream << 48) ^ ((uint64_t)rank << 32) ^ (uint64_t)step);
}

ZSG_FN uint64_t zsg_draw(uint64_t key, uint64_t c)
{
    return zsg_mix64(key + c * ZSG_GOLDEN);
}

ZSG_FN double zsg_bits_to_double(uint64_t b)
{
    union { uint64_t u; double d; } x;
    x.u = b;
    return x.d;
}

ZSG_FN uint64_t zsg_double_to_bits(double d)
{
    union { uint64_t u; double d; } x;
    x.d = d;
    return x.u;
}

/* ln(s) for normal, positive, finite s. */
ZSG_FN double zsg_log(double s)
{
    uint64_t b = zsg_double_to_bits(s);
    int64_t e = (int64_t)((b >> 52) & 0x7FF) - 1023;
    double m = zsg_bits_to_double((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
    if (m > 1.4142135623730951) { m = m * 0.5; e = e + 1; }
    double f = (m - 1.0) / (m + 1.0);
    double f2 = f * f;
    double p = 1.0 / 23.0;
    p = p * f2 + 1.0 / 21.0;
    p = p * f2 + 1.0 / 19.0;
    p = p * f2 + 1.0 / 17.0;
    p = p * f2 + 1.0 / 15.0;
    p = p * f2 + 1.0 / 13.0;
    p = p * f2 + 1.0 / 11.0;
    p = p * f2 + 1.0 / 9.0;
    p = p * f2 + 1.0 / 7.0;
    p = p * f2 + 1.0 / 5.0;
    p = p * f2 + 1.0 / 3.0;
    p = p * f2 + 1.0;
    return (double)e * 0.6931471805599453 + 2.0 * f * p;
}

/* sqrt(r) for normal, positive r well inside float range. */
ZSG_FN double zsg_sqrt(double r, float seed_sqrt)
{
    double y = (double)seed_sqrt;
    y = 0.5 * (y + r / y);
    y = 0.5 * (y + r / y);
    return y;
}

/* The radius factor sqrt(-2 ln s / s) needs a float sqrt for its seed; the
 * includer passes the float square root (IEEE sqrt, correctly rounded). */
#define ZSG_NORMAL_PAIR(key, j, z0, z1, FSQRT)                                  \
    do {                                                                        \
        (z0) = 0.0; (z1) = 0.0;                                                 \
        for (uint64_t a_ = 0; a_ < 64; ++a_) {                                   \
            uint64_t h_ = zsg_draw((key), (uint64_t)(j) * 64u + a_);            \
            double u_ = (double)(int64_t)(h_ >> 40) * (1.0 / 8388608.0) - 1.0;  \
            double v_ = (double)(int64_t)((h_ >> 16) & 0xFFFFFFull)             \
                        * (1.0 / 8388608.0) - 1.0;                              \
            double s_ = u_ * u_ + v_ * v_;                                      \
            if (s_ < 1.0 && s_ > 0.0) {                                         \
                double r_ = -2.0 * zsg_log(s_) / s_;                            \
                double f_ = zsg_sqrt(r_, FSQRT((float)r_));                     \
                (z0) = u_ * f_; (z1) = v_ * f_;                                 \
                break;                                                          \
            }                                                                   \
        }                                                                       \
    } while (0)

/* Truncation toward zero to fp32 / bf16 bit patterns. */
ZSG_FN uint32_t zsg_trunc_f32(double x)
{
    uint64_t b = zsg_double_to_bits(x);
    uint32_t sign = (uint32_t)(b >> 63) << 31;
    int64_t e = (int64_t)((b >> 52) & 0x7FF) - 1023;
    if (e < -126) return sign;                         /* below normal range */
    if (e > 127) return sign | 0x7F7FFFFFu;            /* clamp (never hit) */
    return sign | ((uint32_t)(e + 127) << 23) | (uint32_t)((b >> 29) & 0x7FFFFFu);
}

ZSG_FN uint16_t zsg_trunc_bf16(double x)
{
    return (uint16_t)(zsg_trunc_f32(x) >> 16);
}

/* Stream ids of the workload tensors.  Gradient streams are per (rank, step);
 * state streams use rank = unit index, step = 0. */
#define ZSG_STREAM_MASTER      1u
#define ZSG_STREAM_EXP_AVG     2u
#define ZSG_STREAM_EXP_AVG_SQ  3u
#define ZSG_STREAM_GRAD        4u
#define ZSG_SUBSTREAM_MASK     0x8000u   /* outlier Bernoulli draws */
#define ZSG_SUBSTREAM_OUTLIER  0x4000u   /* outlier values */

#endif
