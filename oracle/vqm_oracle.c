/*
 * vqm_oracle.c — plain single-threaded CPU definition of float_ssim and
 * MS-SSIM.  TEST INFRASTRUCTURE ONLY: the yardstick for the HIP library,
 * never part of it.  See vqm_oracle.h for the sources, readings and pins.
 *
 * Written for a reader checking it against the pages by eye: no blocking, no
 * fusion, no reordering beyond what each definition states.
 */
#include "vqm_oracle.h"

#include <errno.h>
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* Every float expression must round to its own type (no x87 excess
 * precision); contraction is switched off on the compile line. */
_Static_assert(FLT_EVAL_METHOD == 0, "oracle needs FLT_EVAL_METHOD == 0");

/* 11-tap Gaussian window, sigma 1.5, normalised to sum 1 (reading: the pages
 * name only "the 11x11 Gaussian"; sigma 1.5 is the SSIM definition). */
#define WIN 11
#define WIN_HALF 5
#define SIGMA 1.5

/* Dynamic range L = 255 (samples are on the 8-bit scale at every depth). */
#define SSIM_C1 ((0.01 * 255.0) * (0.01 * 255.0))
#define SSIM_C2 ((0.03 * 255.0) * (0.03 * 255.0))

static const double MS_EXPONENT[5] = {0.0448, 0.2856, 0.3001, 0.2363, 0.1333};

static int check_frame_args(const void *a, const void *b, int w, int h, int bpc)
{
    if (!a || !b || w <= 0 || h <= 0 || bpc < 8 || bpc > 16)
        return -EINVAL;
    if ((int64_t)w * (int64_t)h > (int64_t)INT_MAX)
        return -EINVAL;
    return 0;
}

int vqm_oracle_scale(int w, int h)
{
    int m = w < h ? w : h;
    double r = round((double)m / 256.0); /* C round: half away from zero */
    int s = (int)r;
    return s < 1 ? 1 : s;
}

float vqm_oracle_tap(int scale)
{
    return 1.0f / (float)(scale * scale);
}

int vqm_oracle_decimated_dim(int n, int scale)
{
    if (n <= 0 || scale <= 0)
        return -EINVAL;
    return (n + scale - 1) / scale;
}

/* Raw sample at index i of a plane of the given depth, as an integer. */
static unsigned raw_at(const void *raw, int bpc, size_t i)
{
    if (bpc == 8)
        return ((const uint8_t *)raw)[i];
    return ((const uint16_t *)raw)[i];
}

int vqm_oracle_sample_plane(const void *raw, int w, int h, int bpc, float *out)
{
    int rc = check_frame_args(raw, out, w, h, bpc);
    if (rc)
        return rc;
    const float unit = ldexpf(1.0f, -(bpc - 8));
    for (size_t i = 0; i < (size_t)w * (size_t)h; i++)
        out[i] = (float)raw_at(raw, bpc, i) * unit;
    return 0;
}

/* Half-sample symmetric extension: -1 -> 0, n -> n-1; reflect again while
 * still outside (only reachable for planes smaller than the window). */
static int sym(int i, int n)
{
    while (i < 0 || i >= n) {
        if (i < 0)
            i = -i - 1;
        else
            i = 2 * n - i - 1;
    }
    return i;
}

int vqm_oracle_decimate(const void *raw, int w, int h, int bpc, int scale, float *out)
{
    int rc = check_frame_args(raw, out, w, h, bpc);
    if (rc)
        return rc;
    if (scale < 1)
        return -EINVAL;
    const int ow = vqm_oracle_decimated_dim(w, scale);
    const int oh = vqm_oracle_decimated_dim(h, scale);
    const float tap = vqm_oracle_tap(scale);
    const float unit = ldexpf(1.0f, -(bpc - 8));
    const int lo = -(scale / 2);
    const int hi = scale - 1 - scale / 2;
    for (int Y = 0; Y < oh; Y++) {
        for (int X = 0; X < ow; X++) {
            double acc = 0.0;
            for (int j = lo; j <= hi; j++) {
                int yy = sym(Y * scale + j, h);
                for (int i = lo; i <= hi; i++) {
                    int xx = sym(X * scale + i, w);
                    float v = (float)raw_at(raw, bpc, (size_t)yy * w + xx) * unit;
                    float p = v * tap; /* the fp32 product, rounded once */
                    acc += (double)p;  /* exact for scale <= 128 */
                }
            }
            out[(size_t)Y * ow + X] = (float)acc; /* one rounding to fp32 */
        }
    }
    return 0;
}

static void gaussian_window(double g[WIN])
{
    double sum = 0.0;
    for (int k = 0; k < WIN; k++) {
        double d = (double)(k - WIN_HALF);
        g[k] = exp(-(d * d) / (2.0 * SIGMA * SIGMA));
        sum += g[k];
    }
    for (int k = 0; k < WIN; k++)
        g[k] /= sum;
}

/* The five Gaussian moments at map pixel (x, y), i.e. the window whose top
 * left input sample is (x, y): direct 2-D sums with weights g_i * g_j. */
struct moments {
    double mx, my, exx, eyy, exy;
};

static struct moments window_moments(const float *ref, const float *dis, int w,
                                     const double g[WIN], int x, int y)
{
    struct moments m = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (int j = 0; j < WIN; j++) {
        for (int i = 0; i < WIN; i++) {
            double wij = g[j] * g[i];
            size_t idx = (size_t)(y + j) * w + (size_t)(x + i);
            double a = (double)ref[idx];
            double b = (double)dis[idx];
            m.mx += wij * a;
            m.my += wij * b;
            m.exx += wij * (a * a);
            m.eyy += wij * (b * b);
            m.exy += wij * (a * b);
        }
    }
    return m;
}

int vqm_oracle_ssim_planes(const float *ref, const float *dis, int w, int h,
                           double *score, double *map)
{
    if (!ref || !dis || !score || w <= 0 || h <= 0)
        return -EINVAL;
    if (w < WIN || h < WIN)
        return -ENOTSUP;
    double g[WIN];
    gaussian_window(g);
    const int mw = w - (WIN - 1), mh = h - (WIN - 1);
    double total = 0.0;
    for (int y = 0; y < mh; y++) {
        for (int x = 0; x < mw; x++) {
            struct moments m = window_moments(ref, dis, w, g, x, y);
            double sxx = m.exx - m.mx * m.mx;
            double syy = m.eyy - m.my * m.my;
            double sxy = m.exy - m.mx * m.my;
            /* Numerator and denominator written as mirror images, so that
             * identical planes give exactly 1. */
            double num = (m.mx * m.my + m.mx * m.my + SSIM_C1) * (sxy + sxy + SSIM_C2);
            double den = (m.mx * m.mx + m.my * m.my + SSIM_C1) * (sxx + syy + SSIM_C2);
            double v = num / den;
            if (map)
                map[(size_t)y * mw + x] = v;
            total += v;
        }
    }
    *score = total / ((double)mw * (double)mh);
    return 0;
}

int vqm_oracle_ssim(const void *ref, const void *dis, int w, int h, int bpc, double *score)
{
    int rc = check_frame_args(ref, dis, w, h, bpc);
    if (rc)
        return rc;
    if (!score)
        return -EINVAL;
    const int s = vqm_oracle_scale(w, h);
    const int ow = vqm_oracle_decimated_dim(w, s);
    const int oh = vqm_oracle_decimated_dim(h, s);
    if (s > 128 || ow < WIN || oh < WIN)
        return -ENOTSUP;
    float *dr = malloc(sizeof(float) * (size_t)ow * oh);
    float *dd = malloc(sizeof(float) * (size_t)ow * oh);
    if (!dr || !dd) {
        free(dr);
        free(dd);
        return -ENOMEM;
    }
    rc = vqm_oracle_decimate(ref, w, h, bpc, s, dr);
    if (!rc)
        rc = vqm_oracle_decimate(dis, w, h, bpc, s, dd);
    if (!rc)
        rc = vqm_oracle_ssim_planes(dr, dd, ow, oh, score, NULL);
    free(dr);
    free(dd);
    return rc;
}

int vqm_oracle_msssim_level_maps(const float *ref, const float *dis, int w, int h,
                                 double *l, double *c, double *s)
{
    if (!ref || !dis || w <= 0 || h <= 0)
        return -EINVAL;
    if (w < WIN || h < WIN)
        return -ENOTSUP;
    double g[WIN];
    gaussian_window(g);
    const double c3 = SSIM_C2 / 2.0;
    const int mw = w - (WIN - 1), mh = h - (WIN - 1);
    for (int y = 0; y < mh; y++) {
        for (int x = 0; x < mw; x++) {
            struct moments m = window_moments(ref, dis, w, g, x, y);
            double sxx = m.exx - m.mx * m.mx;
            double syy = m.eyy - m.my * m.my;
            double sxy = m.exy - m.mx * m.my;
            double sx = sqrt(sxx > 0.0 ? sxx : 0.0);
            double sy = sqrt(syy > 0.0 ? syy : 0.0);
            size_t o = (size_t)y * mw + x;
            if (l)
                l[o] = (m.mx * m.my + m.mx * m.my + SSIM_C1) /
                       (m.mx * m.mx + m.my * m.my + SSIM_C1);
            if (c)
                c[o] = (sx * sy + sx * sy + SSIM_C2) / (sx * sx + sy * sy + SSIM_C2);
            if (s)
                s[o] = (sxy + c3) / (sx * sy + c3);
        }
    }
    return 0;
}

int vqm_oracle_downsample(const float *in, int w, int h, float *out)
{
    if (!in || !out || w < 2 || h < 2)
        return -EINVAL;
    const int ow = w / 2, oh = h / 2;
    for (int Y = 0; Y < oh; Y++) {
        for (int X = 0; X < ow; X++) {
            float a = in[(size_t)(2 * Y) * w + 2 * X];
            float b = in[(size_t)(2 * Y) * w + 2 * X + 1];
            float c = in[(size_t)(2 * Y + 1) * w + 2 * X];
            float d = in[(size_t)(2 * Y + 1) * w + 2 * X + 1];
            out[(size_t)Y * ow + X] = ((a + b) + (c + d)) * 0.25f;
        }
    }
    return 0;
}

static double mean_of(const double *v, size_t n)
{
    double t = 0.0;
    for (size_t i = 0; i < n; i++)
        t += v[i];
    return t / (double)n;
}

double vqm_oracle_msssim_combine(const double lcs[15])
{
    const double *L = lcs, *C = lcs + 5, *S = lcs + 10;
    double msv = pow(L[4], MS_EXPONENT[4]);
    for (int j = 0; j < 5; j++) {
        if (!(C[j] > 0.0) || !(S[j] > 0.0))
            return NAN;
        msv *= pow(C[j], MS_EXPONENT[j]) * pow(S[j], MS_EXPONENT[j]);
    }
    return msv;
}

int vqm_oracle_msssim(const void *ref, const void *dis, int w, int h, int bpc,
                      double *score, double *lcs)
{
    int rc = check_frame_args(ref, dis, w, h, bpc);
    if (rc)
        return rc;
    if (!score)
        return -EINVAL;
    if (w / 16 < WIN || h / 16 < WIN)
        return -ENOTSUP;

    const size_t n = (size_t)w * h;
    float *xr = malloc(sizeof(float) * n), *xd = malloc(sizeof(float) * n);
    float *nr = malloc(sizeof(float) * n), *nd = malloc(sizeof(float) * n);
    double *ml = malloc(sizeof(double) * n), *mc = malloc(sizeof(double) * n),
           *ms = malloc(sizeof(double) * n);
    if (!xr || !xd || !nr || !nd || !ml || !mc || !ms) {
        rc = -ENOMEM;
        goto done;
    }
    vqm_oracle_sample_plane(ref, w, h, bpc, xr);
    vqm_oracle_sample_plane(dis, w, h, bpc, xd);

    double L[5], C[5], S[5];
    int lw = w, lh = h;
    for (int j = 0; j < 5; j++) {
        rc = vqm_oracle_msssim_level_maps(xr, xd, lw, lh, ml, mc, ms);
        if (rc)
            goto done;
        size_t m = (size_t)(lw - (WIN - 1)) * (size_t)(lh - (WIN - 1));
        L[j] = mean_of(ml, m);
        C[j] = mean_of(mc, m);
        S[j] = mean_of(ms, m);
        if (j < 4) {
            vqm_oracle_downsample(xr, lw, lh, nr);
            vqm_oracle_downsample(xd, lw, lh, nd);
            float *t;
            t = xr; xr = nr; nr = t;
            t = xd; xd = nd; nd = t;
            lw /= 2;
            lh /= 2;
        }
    }

    double means[15];
    for (int j = 0; j < 5; j++) {
        means[j] = L[j];
        means[5 + j] = C[j];
        means[10 + j] = S[j];
    }
    *score = vqm_oracle_msssim_combine(means);
    if (lcs) {
        for (int k = 0; k < 15; k++)
            lcs[k] = means[k];
    }
done:
    free(xr);
    free(xd);
    free(nr);
    free(nd);
    free(ml);
    free(mc);
    free(ms);
    return rc;
}

double vqm_oracle_db(double ssim)
{
    if (!(ssim < 1.0))
        return ssim >= 1.0 ? INFINITY : NAN;
    return -10.0 * log10(1.0 - ssim);
}

int vqm_oracle_plane_dims(int w, int h, int chroma, int plane, int *pw, int *ph)
{
    if (w <= 0 || h <= 0 || plane < 0 || plane > 2 || chroma < 0 || chroma > 2 || !pw || !ph)
        return -EINVAL;
    int sx = 0, sy = 0;
    if (plane > 0) {
        sx = chroma == 2 ? 0 : 1;
        sy = chroma == 0 ? 1 : 0;
    }
    *pw = sx ? (w + 1) / 2 : w;
    *ph = sy ? (h + 1) / 2 : h;
    return 0;
}
