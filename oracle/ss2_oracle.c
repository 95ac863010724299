/*
 * ss2_oracle.c — plain single-threaded CPU definition of the ssimulacra2
 * per-scale statistics, and of the exact fp32-pair operations a device uses
 * to reach them without fp64.  TEST INFRASTRUCTURE ONLY: the yardstick for
 * the HIP library, never part of it.  See vqm_oracle.h for the sources,
 * readings and pins.
 *
 * "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
 * SYCL", Findings 3 and 4: per pixel and channel the SSIM term 1 - q with
 * q = num_m * num_s / denom_s and the edge ratio
 * (1 + |r2 - mu2|) / (1 + |r1 - mu1|) - 1; six sums per channel (the terms
 * and their fourth powers); the CPU evaluates each term in fp64 and adds the
 * terms one after another.  The pair operations follow the published
 * error-free transformations: Knuth's TwoSum, the FMA form of Dekker's
 * TwoProduct, and double-word division by two correctly rounded partial
 * quotients (the page's ff_div).
 */
#include "vqm_oracle.h"

#include <errno.h>
#include <float.h>
#include <math.h>
#include <stddef.h>

_Static_assert(FLT_EVAL_METHOD == 0, "oracle needs FLT_EVAL_METHOD == 0");

/* The SSIM variant's stabilising constant (reading: the published
 * ssimulacra2 uses one constant, 0.0009, in the structure term only). */
#define SS2_C2 0.0009f

/* ---------------------------------------------------------------- pairs */

void vqm_oracle_two_sum(float a, float b, float out[2])
{
    float s = a + b;
    float bb = s - a;
    float e = (a - (s - bb)) + (b - bb);
    out[0] = s;
    out[1] = e;
}

void vqm_oracle_two_prod(float a, float b, float out[2])
{
    float p = a * b;
    out[0] = p;
    out[1] = fmaf(a, b, -p); /* exact: a*b - p is representable */
}

/* |a| >= |b| (or a == 0): s + e == a + b exactly. */
static void fast_two_sum(float a, float b, float out[2])
{
    float s = a + b;
    out[0] = s;
    out[1] = b - (s - a);
}

void vqm_oracle_ff_add(const float a[2], const float b[2], float out[2])
{
    float s[2], t[2], v[2];
    vqm_oracle_two_sum(a[0], b[0], s);
    vqm_oracle_two_sum(a[1], b[1], t);
    float c = s[1] + t[0];
    fast_two_sum(s[0], c, v);
    float w = t[1] + v[1];
    fast_two_sum(v[0], w, out);
}

void vqm_oracle_ff_mul(const float a[2], const float b[2], float out[2])
{
    float p[2];
    vqm_oracle_two_prod(a[0], b[0], p);
    float t = a[0] * b[1];
    t = fmaf(a[1], b[0], t);
    float e = p[1] + t;
    fast_two_sum(p[0], e, out);
}

void vqm_oracle_ff_div(const float a[2], const float b[2], float out[2])
{
    float q1 = a[0] / b[0];       /* first correctly rounded partial quotient */
    float p[2];
    vqm_oracle_two_prod(q1, b[0], p);
    float r = (a[0] - p[0]) - p[1]; /* a - q1 * b, to about 2^-48 relative */
    r = r + a[1];
    r = r - q1 * b[1];
    float q2 = r / b[0];          /* second correctly rounded partial quotient */
    fast_two_sum(q1, q2, out);
}

/* ------------------------------------------------------- the definition */

int vqm_oracle_ss2_channel_sums(const float *img1, const float *img2, const float *mu1, const float *mu2,
                                const float *s11, const float *s22, const float *s12, int w, int h,
                                double sums[6])
{
    if (!img1 || !img2 || !mu1 || !mu2 || !s11 || !s22 || !s12 || !sums || w <= 0 || h <= 0)
        return -EINVAL;
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (size_t i = 0; i < (size_t)w * (size_t)h; i++) {
        /* the fp32 steps, in the order written (no contraction) */
        float m1 = mu1[i], m2 = mu2[i];
        float dm = m1 - m2;
        float num_m = 1.0f - dm * dm;
        float mu12 = m1 * m2;
        float num_s = 2.0f * (s12[i] - mu12) + SS2_C2;
        float mu11 = m1 * m1, mu22 = m2 * m2;
        float denom_s = (s11[i] - mu11) + (s22[i] - mu22) + SS2_C2;
        /* the SSIM term in fp64: the product of two floats is exact there */
        double d = 1.0 - ((double)num_m * (double)num_s) / (double)denom_s;
        if (d < 0.0)
            d = 0.0;
        double d2 = d * d;
        acc[0] += d;
        acc[1] += d2 * d2;
        /* the edge ratio, from fp32 differences */
        float a2 = fabsf(img2[i] - m2);
        float a1 = fabsf(img1[i] - m1);
        double e = (1.0 + (double)a2) / (1.0 + (double)a1) - 1.0;
        double art = e > 0.0 ? e : 0.0;
        double det = e < 0.0 ? -e : 0.0;
        double art2 = art * art, det2 = det * det;
        acc[2] += art;
        acc[3] += art2 * art2;
        acc[4] += det;
        acc[5] += det2 * det2;
    }
    for (int k = 0; k < 6; k++)
        sums[k] = acc[k];
    return 0;
}
