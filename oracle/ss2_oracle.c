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
 *
 * The per-scale chain (Findings 2 and 7): per scale the three multiplies,
 * five blurs (a recursive filter along every row, then along every column),
 * the six sums per channel, and the 2x2 downsample to the next scale, all in
 * fp32 with no contraction, as the page's CPU extractor computes them.
 */
#include "vqm_oracle.h"

#include <errno.h>
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

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

/* ------------------------------------------------- the per-scale chain */

/* One line through the third-order recursion, causal then anticausal, the
 * filter at rest outside the line.  Each product is its own rounded fp32
 * value, and each sum adds the terms from the oldest state to the newest. */
static void iir_line(const float *x, long sx, float *y, long sy, int n, const float coef[4], float *w)
{
    const float B = coef[0], a1 = coef[1], a2 = coef[2], a3 = coef[3];
    float p1 = 0.0f, p2 = 0.0f, p3 = 0.0f; /* w[i-1], w[i-2], w[i-3] */
    for (int i = 0; i < n; i++) {
        float in = B * x[(long)i * sx];
        float t3 = a3 * p3;
        float t2 = a2 * p2;
        float t1 = a1 * p1;
        float v = ((in + t3) + t2) + t1;
        w[i] = v;
        p3 = p2;
        p2 = p1;
        p1 = v;
    }
    float q1 = 0.0f, q2 = 0.0f, q3 = 0.0f; /* y[i+1], y[i+2], y[i+3] */
    for (int i = n - 1; i >= 0; i--) {
        float in = B * w[i];
        float t3 = a3 * q3;
        float t2 = a2 * q2;
        float t1 = a1 * q1;
        float v = ((in + t3) + t2) + t1;
        y[(long)i * sy] = v;
        q3 = q2;
        q2 = q1;
        q1 = v;
    }
}

int vqm_oracle_iir_line(const float *x, int n, const float coef[4], float *y)
{
    if (!x || !y || !coef || n <= 0)
        return -EINVAL;
    float *w = malloc((size_t)n * sizeof(float));
    if (!w)
        return -ENOMEM;
    iir_line(x, 1, y, 1, n, coef, w);
    free(w);
    return 0;
}

int vqm_oracle_ss2_blur(const float *in, int w, int h, const float coef[4], float *out)
{
    if (!in || !out || !coef || w <= 0 || h <= 0)
        return -EINVAL;
    size_t n = (size_t)w * (size_t)h;
    float *rows = malloc(n * sizeof(float));
    float *line = malloc((size_t)(w > h ? w : h) * sizeof(float));
    if (!rows || !line) {
        free(rows);
        free(line);
        return -ENOMEM;
    }
    for (int r = 0; r < h; r++) /* every row first */
        iir_line(in + (size_t)r * w, 1, rows + (size_t)r * w, 1, w, coef, line);
    for (int c = 0; c < w; c++) /* then every column of the row pass's output */
        iir_line(rows + c, w, out + c, w, h, coef, line);
    free(rows);
    free(line);
    return 0;
}

void vqm_oracle_ss2_downsampled_dim(int w, int h, int *ow, int *oh)
{
    *ow = (w + 1) / 2;
    *oh = (h + 1) / 2;
}

int vqm_oracle_ss2_downsample(const float *in, int w, int h, float *out)
{
    if (!in || !out || w <= 0 || h <= 0)
        return -EINVAL;
    int ow, oh;
    vqm_oracle_ss2_downsampled_dim(w, h, &ow, &oh);
    for (int y = 0; y < oh; y++) {
        int r0 = 2 * y, r1 = 2 * y + 1 < h ? 2 * y + 1 : h - 1;
        for (int x = 0; x < ow; x++) {
            int c0 = 2 * x, c1 = 2 * x + 1 < w ? 2 * x + 1 : w - 1;
            float a = in[(size_t)r0 * w + c0], b = in[(size_t)r0 * w + c1];
            float c = in[(size_t)r1 * w + c0], d = in[(size_t)r1 * w + c1];
            out[(size_t)y * ow + x] = ((a + b) + (c + d)) * 0.25f;
        }
    }
    return 0;
}

int vqm_oracle_ss2_cascade_coefficients(double sigma, float coef[4])
{
    if (!coef || !(sigma > 0.0) || !(sigma < 1e6))
        return -EINVAL;
    /* Three symmetric exponential smoothers, each a first-order causal pass
     * and its anticausal mirror with pole p: one has variance
     * 2p / (1 - p)^2, three have 6p / (1 - p)^2 = sigma^2.  Solved for the
     * root in (0, 1): s^2 p^2 - (2 s^2 + 6) p + s^2 = 0. */
    double s2 = sigma * sigma;
    double p = ((s2 + 3.0) - sqrt(6.0 * s2 + 9.0)) / s2;
    double g = 1.0 - p;
    coef[0] = (float)(g * g * g); /* B: the cube of one pass's gain */
    coef[1] = (float)(3.0 * p);   /* (1 - p z^-1)^3 = 1 - 3p z^-1 + 3p^2 z^-2 - p^3 z^-3 */
    coef[2] = (float)(-3.0 * p * p);
    coef[3] = (float)(p * p * p);
    return 0;
}

int vqm_oracle_ss2_chain(const float *const *ref, const float *const *dis, int nch, int w, int h, int nscales,
                         const float coef[4], double *sums)
{
    if (!ref || !dis || !coef || !sums || nch < 1 || nch > 3 || w <= 0 || h <= 0 || nscales < 1 ||
        nscales > 6)
        return -EINVAL;
    for (int c = 0; c < nch; c++)
        if (!ref[c] || !dis[c])
            return -EINVAL;
    size_t n0 = (size_t)w * (size_t)h;
    /* per channel: the scale's two images (copies, downsampled in place of
     * the previous scale's), three products and five blurred planes */
    float *buf = malloc(n0 * sizeof(float) * (size_t)(2 * nch + 3 + 5));
    if (!buf)
        return -ENOMEM;
    float *img = buf;                     /* 2 * nch planes */
    float *prod = buf + 2 * (size_t)nch * n0; /* aa, bb, ab */
    float *blr = prod + 3 * n0;          /* mu1, mu2, s11, s22, s12 */
    float *tmp = malloc(n0 * sizeof(float));
    if (!tmp) {
        free(buf);
        return -ENOMEM;
    }
    for (int c = 0; c < nch; c++) {
        memcpy(img + (2 * (size_t)c) * n0, ref[c], n0 * sizeof(float));
        memcpy(img + (2 * (size_t)c + 1) * n0, dis[c], n0 * sizeof(float));
    }
    int sw = w, sh = h, rc = 0;
    for (int s = 0; s < nscales && rc == 0; s++) {
        if (s > 0) { /* the next scale's images: 2x2 means of this one's */
            int nw, nh;
            vqm_oracle_ss2_downsampled_dim(sw, sh, &nw, &nh);
            for (int k = 0; k < 2 * nch; k++) {
                float *p = img + (size_t)k * n0;
                vqm_oracle_ss2_downsample(p, sw, sh, tmp);
                memcpy(p, tmp, (size_t)nw * nh * sizeof(float));
            }
            sw = nw;
            sh = nh;
        }
        size_t n = (size_t)sw * (size_t)sh;
        for (int c = 0; c < nch && rc == 0; c++) {
            const float *a = img + (2 * (size_t)c) * n0, *b = img + (2 * (size_t)c + 1) * n0;
            float *aa = prod, *bb = prod + n0, *ab = prod + 2 * n0;
            for (size_t i = 0; i < n; i++) { /* the three multiplies */
                aa[i] = a[i] * a[i];
                bb[i] = b[i] * b[i];
                ab[i] = a[i] * b[i];
            }
            const float *src[5] = {a, b, aa, bb, ab};
            for (int k = 0; k < 5 && rc == 0; k++)
                rc = vqm_oracle_ss2_blur(src[k], sw, sh, coef, blr + (size_t)k * n0);
            if (rc == 0)
                rc = vqm_oracle_ss2_channel_sums(a, b, blr, blr + n0, blr + 2 * n0, blr + 3 * n0, blr + 4 * n0, sw,
                                                 sh, sums + ((size_t)s * nch + c) * 6);
        }
    }
    free(tmp);
    free(buf);
    return rc;
}
