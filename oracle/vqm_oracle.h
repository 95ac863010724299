/*
 * vqm_oracle.h — plain, slow, single-threaded CPU definition of per-frame
 * float_ssim and 5-scale MS-SSIM.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the yardstick the HIP path is
 * held against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it; the product path never calls it, and it shares no
 * code, header, table or constant with the HIP library.
 *
 * Sources (page title, section):
 *   [ADR-1405] "ADR-1405: float_ssim_hip decimates on the device,
 *              bit-identical to the CPU" — Context, Decision 1–4,
 *              Alternatives considered, Consequences.
 *   [R-1363]   "Research-1363: Device-resident ssimulacra2 and a single-wait
 *              MS-SSIM on SYCL" — Findings 4 and 6.
 *
 * Numerics: exact where the method is exact (decimation, pyramid); fp64
 * everywhere else, except the fp32 steps the pages fix (the tap weight, the
 * window products and the single rounding of each decimated sample).  Built
 * with -O2 -std=c11 -ffp-contract=off on x86-64 (FLT_EVAL_METHOD == 0).
 *
 * Readings of points the pages leave open are listed with each function.
 * Every function returns 0 or a negative errno (-EINVAL, -ENOTSUP, -ENOMEM).
 *
 * Pins (what each part is checked against, outside this library):
 *   scale rule        — the sizes the ADR prints (1 below 384 px, 4 at 1080p,
 *                       8 at 2160p) and 481 -> 2.
 *   tap               — exact rational 1/s^2 rounded to fp32.
 *   decimation        — an exact-rational (Fraction) brute force; the
 *                       power-of-two closed form; the ADR's fp32-accumulation
 *                       negative control (scales 3,5,6,7,9,10 differ, 2,4,8 do
 *                       not); the exactness bound at scale 128.
 *   ssim              — identity (exactly 1), the constant-plane closed form,
 *                       a 50-digit mpmath evaluation on 11x11..13x17 planes,
 *                       scipy.ndimage.correlate moments, argument symmetry.
 *   ms-ssim           — identity, the constant-plane closed form L5^b5, the
 *                       pyramid's exactness, mean(l*c*s) at level 1 equal to
 *                       float_ssim at scale 1, a checkerboard that vanishes
 *                       under 2x2 averaging (isolates level 1 and its
 *                       exponent), and a pixel-replicated frame whose levels
 *                       2..5 equal the original's levels 1..4.
 *   ms combine        — each exponent on its own: means of 1 except
 *                       C_j = S_j = 1/2 give 4^-b_j, L_5 = 1/2 gives 2^-b5,
 *                       against the five weights of the published MS-SSIM.
 *   db                — 10, 20, 30 dB at 1 - ssim = 1e-1, 1e-2, 1e-3; the
 *                       ADR's sensitivity 4.34 / (1 - ssim) as a finite
 *                       difference, and its 0.018 dB at 30 dB example.
 *   ss2 sums          — exact rational sums on planes whose fp32 steps are
 *                       exact; identical inputs give six zeros; closed forms
 *                       of constant planes.  Parity with the pages' own
 *                       ssimulacra2 scores is unpinned (no fixture here).
 *   pairs             — two_sum and two_prod exact against Fraction; ff_add,
 *                       ff_mul and ff_div within their error bounds.
 *   ss2 blur          — exact rational recursions on dyadic coefficients and
 *                       inputs; the closed-form impulse response of the
 *                       exponential cascade; scipy.signal.lfilter in fp64 on
 *                       random lines and planes, within fp32 rounding.
 *   ss2 downsample    — exact 2x2 means of dyadic samples, odd edges.
 *   ss2 coefficients  — variance sigma^2 and unit gain of the impulse
 *                       response, in closed form and summed.
 *   ss2 chain         — identical inputs give zeros at every scale; an
 *                       independent fp64 numpy/scipy evaluation of the same
 *                       stages within the fp32 chain's rounding.
 */
#ifndef VQM_ORACLE_H
#define VQM_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Decimation factor: max(1, round(min(w, h) / 256)), real division, round
 * half away from zero. [ADR-1405] Context. */
int vqm_oracle_scale(int w, int h);

/* Box tap weight 1.0f / (scale * scale), formed in fp32. [ADR-1405] Decision 1. */
float vqm_oracle_tap(int scale);

/* Decimated extent of one dimension: ceil(n / scale) — one output per
 * sampled position x*scale < n (reading: the page names iqa_decimate_dim()
 * without its formula). Returns -EINVAL for n <= 0 or scale <= 0. */
int vqm_oracle_decimated_dim(int n, int scale);

/* Sample value v = raw * 2^-(bpc-8), i.e. every bit depth mapped onto the
 * 8-bit range (reading: exact in fp32; keeps the 2^-52 window sum below
 * 2^60).  raw: uint8_t when bpc == 8, else uint16_t; w*h samples. */
int vqm_oracle_sample_plane(const void *raw, int w, int h, int bpc, float *out);

/* Exact box low-pass and decimate of one plane. [ADR-1405] Context and
 * Decision 1: output (X, Y) sums, over offsets -scale/2 .. scale-1-scale/2
 * in both directions with half-sample symmetric edges, the fp32 products
 * v * tap; the sum is exact (here a C double, exact for scale <= 128) and is
 * rounded once to fp32.  out: ceil(w/s) x ceil(h/s) floats, row-major,
 * tightly packed.  Any scale >= 1 is accepted (the exactness guarantee, and
 * so bit-identity with other exact methods, holds to 128). */
int vqm_oracle_decimate(const void *raw, int w, int h, int bpc, int scale, float *out);

/* SSIM of two fp32 planes (w x h) with the 11x11 Gaussian (sigma 1.5,
 * normalised), "valid" region only: map (w-10) x (h-10).  Moments as direct
 * 2-D weighted sums in fp64.  Per pixel
 *   ((2 mx my + C1)(2 sxy + C2)) / ((mx^2 + my^2 + C1)(sxx + syy + C2)),
 * C1 = (0.01*255)^2, C2 = (0.03*255)^2; score = fp64 sequential mean.
 * map (optional, may be NULL): (w-10)*(h-10) doubles.
 * Returns -ENOTSUP when w < 11 or h < 11. [ADR-1405] Context, Decision 4. */
int vqm_oracle_ssim_planes(const float *ref, const float *dis, int w, int h,
                           double *score, double *map);

/* float_ssim of one raw frame pair: scale, gate (-ENOTSUP when scale > 128 or
 * a decimated side < 11), sample, decimate, SSIM. [ADR-1405] Context,
 * Decision 1 and 4. */
int vqm_oracle_ssim(const void *ref, const void *dis, int w, int h, int bpc, double *score);

/* One MS-SSIM level: per-pixel luminance, contrast and structure maps over
 * the valid region ((w-10) x (h-10) doubles each; any may be NULL), with
 * sigma = sqrt(max(var, 0)) and C3 = C2 / 2. */
int vqm_oracle_msssim_level_maps(const float *ref, const float *dis, int w, int h,
                                 double *l, double *c, double *s);

/* 2x2 mean in fp32, ((a + b) + (c + d)) * 0.25f, output floor(w/2) x floor(h/2). */
int vqm_oracle_downsample(const float *in, int w, int h, float *out);

/* The MS-SSIM combine of 15 level means (L_1..L_5, C_1..C_5, S_1..S_5):
 *   MS = L5^b5 * prod_{j=1..5} C_j^b_j * S_j^b_j,
 *   b = {0.0448, 0.2856, 0.3001, 0.2363, 0.1333}
 * (reading: the five weights of the published multi-scale SSIM, Wang,
 * Simoncelli and Bovik 2003, which the MS-SSIM workload states; luminance
 * enters at the coarsest level only).  NaN when any C_j or S_j is <= 0
 * (reading: the power of a non-positive mean is not defined). */
double vqm_oracle_msssim_combine(const double lcs[15]);

/* 5-scale MS-SSIM at full resolution (no decimation first):
 *   MS = L5^b5 * prod_{j=1..5} C_j^b_j * S_j^b_j,
 *   b = {0.0448, 0.2856, 0.3001, 0.2363, 0.1333},
 * L_j, C_j, S_j the valid-region means of level j.  NaN when any C_j or S_j
 * is <= 0.  Gate: -ENOTSUP when floor(w/16) < 11 or floor(h/16) < 11.
 * lcs (optional, may be NULL): 15 doubles, L_1..L_5, C_1..C_5, S_1..S_5.
 * [R-1363] Finding 6 (per-scale l/c/s spans). */
int vqm_oracle_msssim(const void *ref, const void *dis, int w, int h, int bpc,
                      double *score, double *lcs);

/* Size of plane `plane` (0 = Y, 1 = Cb, 2 = Cr) of a w x h picture whose
 * chroma layout is `chroma`: 0 = 4:2:0 (chroma halved both ways), 1 = 4:2:2
 * (halved horizontally), 2 = 4:4:4.  An odd size halves rounding up, so the
 * last chroma sample covers the last luma column or row alone (reading: the
 * pages score Cb and Cr planes of 4:2:0 and 4:2:2 pictures, the Netflix pair
 * and its 4:2:2 conversion among them, but give no formula for their sizes).
 * Each plane is scored on its own, with its own decimation scale.
 * [R-1363] Finding 6 (enable_chroma); "Research-1369: SYCL psnr_hvs,
 * motion_v2 and psnr at 4K", section 4.  Returns -EINVAL for bad arguments. */
int vqm_oracle_plane_dims(int w, int h, int chroma, int plane, int *pw, int *ph);

/* A score in decibels, the enable_db form of float_ssim:
 *   db = -10 log10(1 - ssim),  +inf when ssim >= 1 (reading: the page gives
 * only the form's sensitivity, 4.34 / (1 - ssim) dB per unit of ssim, which is
 * the derivative of this function; identical planes have no finite value).
 * [ADR-1405] Consequences. */
double vqm_oracle_db(double ssim);

/* ---------------------------------------------------------------------
 * ssimulacra2: the per-scale statistics and exact fp32 pairs
 * ("Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
 * SYCL", Findings 3-5).  Source: ss2_oracle.c.
 *
 * The six sums of one channel at one scale, from seven w x h fp32 planes:
 * the two images r1, r2, their blurred means mu1, mu2, and the blurred
 * products s11 = blur(r1 r1), s22 = blur(r2 r2), s12 = blur(r1 r2).  Per
 * pixel, in fp32 and in this order (readings: the page names num_m, num_s,
 * denom_s and the term 1 - q without defining them; these are the published
 * ssimulacra2 definitions, with its one constant C2 = 0.0009f):
 *   num_m   = 1 - (mu1 - mu2)^2
 *   num_s   = 2 (s12 - mu1 mu2) + C2
 *   denom_s = (s11 - mu1^2) + (s22 - mu2^2) + C2
 * then in fp64, as the page's CPU extractor does (Finding 3):
 *   d   = max(1 - num_m num_s / denom_s, 0)       (reading: the published
 *         metric clamps the SSIM deficit at 0)
 *   e   = (1 + |r2 - mu2|) / (1 + |r1 - mu1|) - 1  (Finding 4, as printed;
 *         each |.| of an fp32 difference)
 *   art = max(e, 0), det = max(-e, 0)
 * sums[] = { sum d, sum d^4, sum art, sum art^4, sum det, sum det^4 }, each
 * an fp64 sum of the terms one after another in row-major order (Finding 3:
 * the CPU adds the fp64 terms sequentially).
 * Returns -EINVAL for NULL pointers or a non-positive size. */
int vqm_oracle_ss2_channel_sums(const float *img1, const float *img2, const float *mu1, const float *mu2,
                                const float *s11, const float *s22, const float *s12, int w, int h,
                                double sums[6]);

/* Error-free transformations and fp32-pair ("double-float") arithmetic, the
 * tools of Finding 4.  A pair (hi, lo) stands for the real number hi + lo.
 *   two_sum(a, b):   s = fl(a + b), e = a + b - s exactly (Knuth).
 *   two_prod(a, b):  p = fl(a b), e = a b - p exactly, by one fused
 *                    multiply-add (exact barring underflow).
 *   ff_add(a, b):    a + b as a pair, relative error below about 3 * 2^-48.
 *   ff_mul(a, b):    a b as a pair, relative error below about 7 * 2^-48.
 *   ff_div(a, b):    a / b from two correctly rounded fp32 partial quotients
 *                    (the page's ff_div), relative error about 2^-46. */
void vqm_oracle_two_sum(float a, float b, float out[2]);
void vqm_oracle_two_prod(float a, float b, float out[2]);
void vqm_oracle_ff_add(const float a[2], const float b[2], float out[2]);
void vqm_oracle_ff_mul(const float a[2], const float b[2], float out[2]);
void vqm_oracle_ff_div(const float a[2], const float b[2], float out[2]);

/* The per-scale chain that feeds those sums (Finding 7's stages after the
 * colour transform: three multiplies, horizontal and vertical blur passes,
 * the sums, the downsample; Finding 2: each stage reproducible bit for bit
 * in fp32 with contraction off and every product its own rounded value).
 *
 * The blur (reading: the pages name a recursive Gaussian walked along each
 * row, then each column, without its coefficients or edges).  A third-order
 * recursion with caller coefficients coef = {B, a1, a2, a3}, at rest
 * outside the line (zero state), causal then anticausal:
 *   w[i] = ((B x[i] + a3 w[i-3]) + a2 w[i-2]) + a1 w[i-1],   i = 0..n-1
 *   y[i] = ((B w[i] + a3 y[i+3]) + a2 y[i+2]) + a1 y[i+1],   i = n-1..0
 * each product rounded to fp32 on its own, the sum from the oldest state to
 * the newest.  ss2_blur applies it to every row, then to every column of
 * the row pass's fp32 output.
 *
 * The downsample (reading: only "downsample_2x2" is named): a w x h plane
 * to ceil(w/2) x ceil(h/2), out = ((a + b) + (c + d)) * 0.25f over the 2x2
 * block, a and b from the upper row, with the last column and row repeated
 * when the size is odd.
 *
 * The chain, per scale s = 0..nscales-1 (nscales 1..6; reading: the
 * published ssimulacra2 has six scales), for each of nch (1..3) channels of
 * w x h fp32 planes ref[c], dis[c] (scale 0 as given, each later scale the
 * downsample of the one before): aa = a a, bb = b b, ab = a b; the five
 * blurs mu1, mu2, s11, s22, s12 of a, b, aa, bb, ab; then
 * ss2_channel_sums(a, b, mu1, mu2, s11, s22, s12) into
 * sums[(s * nch + c) * 6 ..].  The planes are whatever the colour transform
 * gives (reading: the pages fix none of its constants, so the chain starts
 * from the transformed planes and downsamples them).
 *
 * cascade_coefficients(sigma): the coefficients of three symmetric
 * exponential smoothers in series, {(1-p)^3, 3p, -3p^2, p^3} with p the
 * root in (0, 1) of 6p / (1-p)^2 = sigma^2, so the filter's impulse
 * response has variance sigma^2 (reading: one choice of recursive Gaussian
 * among many; the chain takes any coefficients). */
int vqm_oracle_iir_line(const float *x, int n, const float coef[4], float *y);
int vqm_oracle_ss2_blur(const float *in, int w, int h, const float coef[4], float *out);
void vqm_oracle_ss2_downsampled_dim(int w, int h, int *ow, int *oh);
int vqm_oracle_ss2_downsample(const float *in, int w, int h, float *out);
int vqm_oracle_ss2_cascade_coefficients(double sigma, float coef[4]);
int vqm_oracle_ss2_chain(const float *const *ref, const float *const *dis, int nch, int w, int h, int nscales,
                         const float coef[4], double *sums);

#ifdef __cplusplus
}
#endif
#endif
