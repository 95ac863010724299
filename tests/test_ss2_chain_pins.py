"""Pins of the oracle's ssimulacra2 per-scale chain: the recursive blur, the
2x2 downsample, the filter design and the chain that joins them to the six
sums.

"Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
SYCL", Findings 2 and 7.  Each check holds the oracle against something other
than itself: exact rational recursions, scipy's ``lfilter`` in fp64, closed
forms of the exponential cascade, and an fp64 numpy/scipy evaluation of the
whole chain written here from the stage list.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.signal import lfilter

import oracle


def F(x):
    return Fraction(float(x))


def exact_recursion(x, coef):
    """The zero-state causal, then anticausal, recursion in exact rationals."""
    B, a1, a2, a3 = (F(c) for c in coef)
    n = len(x)
    w = []
    for i in range(n):
        prev = [w[i - k] if i - k >= 0 else Fraction(0) for k in (1, 2, 3)]
        w.append(B * F(x[i]) + a1 * prev[0] + a2 * prev[1] + a3 * prev[2])
    y = [Fraction(0)] * n
    for i in range(n - 1, -1, -1):
        nxt = [y[i + k] if i + k < n else Fraction(0) for k in (1, 2, 3)]
        y[i] = B * w[i] + a1 * nxt[0] + a2 * nxt[1] + a3 * nxt[2]
    return y


def fp64_recursion(x, coef):
    """scipy's direct-form filter in fp64: causal, then the mirrored pass."""
    B, a1, a2, a3 = (float(c) for c in coef)
    den = [1.0, -a1, -a2, -a3]
    w = lfilter([B], den, np.asarray(x, np.float64), axis=-1)
    return lfilter([B], den, w[..., ::-1], axis=-1)[..., ::-1]


def fp64_blur(plane, coef):
    rows = fp64_recursion(plane, coef)
    return fp64_recursion(rows.T, coef).T


# Distinct dyadic coefficients of both signs: every product and sum below is
# exact in fp32, so the oracle must equal the rational recursion exactly, and
# any exchange of a1, a2, a3 changes the result.
DYADIC = (0.5, 0.25, -0.125, 0.0625)
# A stable set with complex poles (0.6 and 0.5 +- 0.3i) and unit gain.
COMPLEX = (0.136, 1.6, -0.94, 0.204)


def _representable(vals):
    return all(F(np.float32(float(v))) == v for v in vals)


@pytest.mark.parametrize("x", [[1], [3, 0], [1, 2, 3], [4, 0, 0, 1], [2, 1, 0, 3, 1], [0, 0, 5, 0, 0, 0]])
def test_recursion_exact_on_dyadic_coefficients(x):
    want = exact_recursion(x, DYADIC)
    assert _representable(want), "fixture must stay exact in fp32"
    got = oracle.iir_line(np.array(x, np.float32), DYADIC)
    assert [F(v) for v in got] == want


@pytest.mark.parametrize("coef", ["cascade0.7", "cascade1.5", "cascade4", "complex"])
@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 301])
def test_recursion_matches_lfilter(coef, n):
    c = COMPLEX if coef == "complex" else oracle.ss2_cascade_coefficients(float(coef[7:]))
    rng = np.random.default_rng(n)
    x = rng.uniform(-1.0, 1.0, n).astype(np.float32)
    got = oracle.iir_line(x, c).astype(np.float64)
    want = fp64_recursion(x.astype(np.float64), np.asarray(c, np.float32))
    # fp32 steps: a few roundings per sample, carried by a filter whose
    # absolute impulse response sums to at most ~2 here
    assert np.max(np.abs(got - want)) <= 2e-6 * max(1.0, np.max(np.abs(x)))


def test_cascade_impulse_response_closed_form():
    # Three exponential smoothers in series: the causal response is
    # (1-p)^3 C(k+2, 2) p^k; on a line at rest the two passes give
    # y[i] = sum_j h[j - i] h[j - m] over j >= max(i, m) inside the line.
    sigma = 1.5
    s2 = sigma * sigma
    roots = np.roots([s2, -(2 * s2 + 6), s2])
    p = float(roots[(roots > 0) & (roots < 1)][0])
    n, m = 120, 47
    h = np.array([(1 - p) ** 3 * math.comb(k + 2, 2) * p ** k for k in range(n)])
    want = np.array([sum(h[j - i] * h[j - m] for j in range(max(i, m), n)) for i in range(n)])
    x = np.zeros(n, np.float32)
    x[m] = 1.0
    got = oracle.iir_line(x, oracle.ss2_cascade_coefficients(sigma))
    assert np.max(np.abs(got - want)) < 2e-7


@pytest.mark.parametrize("sigma", [0.5, 1.0, 1.5, 3.0, 8.0])
def test_cascade_coefficients_give_variance_sigma_squared(sigma):
    c = oracle.ss2_cascade_coefficients(sigma).astype(np.float64)
    # unit gain: B = 1 - a1 - a2 - a3 up to fp32 rounding of each coefficient
    assert abs(c[0] - (1 - c[1] - c[2] - c[3])) < 4e-7
    # all three poles at one real p in (0, 1): a1 = 3p, a2 = -3p^2, a3 = p^3
    poles = np.roots([1.0, -c[1], -c[2], -c[3]])
    assert np.all(np.abs(poles) < 1) and np.max(np.abs(poles.imag)) < 2e-2
    # the impulse response (fp64 lfilter on a long line) has variance sigma^2
    n = int(40 * sigma + 60)
    x = np.zeros(2 * n + 1)
    x[n] = 1.0
    y = fp64_recursion(x, c)
    k = np.arange(-n, n + 1)
    # the summed response equals the closed-form gain of the rounded
    # coefficients, (B / (1 - a1 - a2 - a3))^2, which is 1 up to the
    # coefficients' fp32 rounding, amplified by 1 / (1 - p)^3
    gain = (c[0] / (1.0 - c[1] - c[2] - c[3])) ** 2
    assert abs(y.sum() - gain) < 1e-9
    assert abs(gain - 1.0) < 1e-4
    assert abs((k * k * y).sum() - sigma * sigma) < 1e-4 * sigma * sigma


def test_cascade_coefficients_refuse_bad_sigma():
    for s in (0.0, -1.0, float("nan")):
        with pytest.raises(oracle.OracleError):
            oracle.ss2_cascade_coefficients(s)


@pytest.mark.parametrize("shape", [(1, 1), (1, 9), (9, 1), (23, 37), (64, 17)])
def test_blur_matches_fp64_rows_then_columns(shape):
    rng = np.random.default_rng(shape[0] * 100 + shape[1])
    plane = rng.uniform(0.0, 1.0, shape).astype(np.float32)
    for c in (oracle.ss2_cascade_coefficients(1.5), COMPLEX):
        got = oracle.ss2_blur(plane, c).astype(np.float64)
        want = fp64_blur(plane.astype(np.float64), np.asarray(c, np.float32))
        assert np.max(np.abs(got - want)) <= 4e-6


def test_blur_is_rows_then_columns_of_the_line_recursion():
    # The order of the passes decides fp32's rounding (exact arithmetic
    # would not see it): rows first, each column of the rounded row output.
    rng = np.random.default_rng(7)
    plane = rng.uniform(0.0, 1.0, (19, 26)).astype(np.float32)
    c = oracle.ss2_cascade_coefficients(1.5)
    rows = np.stack([oracle.iir_line(r, c) for r in plane])
    want = np.stack([oracle.iir_line(col, c) for col in rows.T]).T
    assert np.array_equal(oracle.ss2_blur(plane, c), want)
    cols_first = np.stack([oracle.iir_line(col, c) for col in plane.T]).T
    cols_first = np.stack([oracle.iir_line(r, c) for r in cols_first])
    assert not np.array_equal(want, cols_first)  # the order is visible


def _clamped_mean(p, y, x):
    h, w = p.shape
    r1, c1 = min(2 * y + 1, h - 1), min(2 * x + 1, w - 1)
    return (F(p[2 * y, 2 * x]) + F(p[2 * y, c1]) + F(p[r1, 2 * x]) + F(p[r1, c1])) / 4


@pytest.mark.parametrize("shape", [(1, 1), (2, 2), (3, 5), (6, 7), (8, 8), (1, 6), (7, 1)])
def test_downsample_exact_means(shape):
    rng = np.random.default_rng(sum(shape))
    p = rng.integers(0, 256, shape).astype(np.float32)
    got = oracle.ss2_downsample(p)
    h, w = shape
    assert got.shape == (-(-h // 2), -(-w // 2))
    for y in range(got.shape[0]):
        for x in range(got.shape[1]):
            assert F(got[y, x]) == _clamped_mean(p, y, x)


def test_downsampled_dims_round_up():
    assert oracle.ss2_downsampled_dim(3840, 2160) == (1920, 1080)
    assert oracle.ss2_downsampled_dim(853, 481) == (427, 241)
    assert oracle.ss2_downsampled_dim(1, 1) == (1, 1)


# ------------------------------------------------------------------ the chain


def _xyb_like(seed, w, h, nch=3):
    """Smooth fields of XYB-like ranges and a noisy distorted copy."""
    rng = np.random.default_rng(seed)
    yy, xx = np.mgrid[0:h, 0:w]
    ref, dis = [], []
    for c, (off, amp) in enumerate([(0.0, 0.02), (0.45, 0.3), (0.4, 0.25)][:nch]):
        f = off + amp * np.sin(xx * (0.07 + 0.05 * c) + yy * 0.11) * np.cos(yy * (0.05 + 0.03 * c))
        f = f + amp * 0.1 * rng.standard_normal((h, w))
        ref.append(f.astype(np.float32))
        dis.append((f + amp * 0.05 * rng.standard_normal((h, w))).astype(np.float32))
    return ref, dis


def fp64_chain(ref, dis, nscales, coef):
    """The stages of Finding 7 from the fp32 input planes, all in fp64."""
    c2 = float(np.float32(0.0009))
    imgs = [(r.astype(np.float64), d.astype(np.float64)) for r, d in zip(ref, dis)]
    out = np.zeros((nscales, len(ref), 6))
    for s in range(nscales):
        if s > 0:
            def down(p):
                h, w = p.shape
                q = np.pad(p, ((0, h % 2), (0, w % 2)), mode="edge")
                return 0.25 * (q[0::2, 0::2] + q[0::2, 1::2] + q[1::2, 0::2] + q[1::2, 1::2])
            imgs = [(down(a), down(b)) for a, b in imgs]
        for ch, (a, b) in enumerate(imgs):
            mu1, mu2, s11, s22, s12 = (fp64_blur(p, coef) for p in (a, b, a * a, b * b, a * b))
            num_m = 1.0 - (mu1 - mu2) ** 2
            num_s = 2.0 * (s12 - mu1 * mu2) + c2
            den_s = (s11 - mu1 * mu1) + (s22 - mu2 * mu2) + c2
            d = np.maximum(1.0 - num_m * num_s / den_s, 0.0)
            e = (1.0 + np.abs(b - mu2)) / (1.0 + np.abs(a - mu1)) - 1.0
            art, det = np.maximum(e, 0.0), np.maximum(-e, 0.0)
            out[s, ch] = [d.sum(), (d ** 4).sum(), art.sum(), (art ** 4).sum(), det.sum(), (det ** 4).sum()]
    return out


@pytest.mark.parametrize("w,h,nscales", [(40, 29, 4), (17, 16, 6), (33, 9, 3)])
def test_chain_matches_fp64_evaluation(w, h, nscales):
    ref, dis = _xyb_like(w * h, w, h)
    coef = oracle.ss2_cascade_coefficients(1.5)
    got = oracle.ss2_chain(ref, dis, nscales, coef)
    want = fp64_chain(ref, dis, nscales, np.asarray(coef, np.float32))
    # fp32 blurred moments move 1 - q (a difference of nearly equal numbers)
    # by up to ~1e-7 per pixel, a large share of the small deficits of the
    # coarse scales; the edge sums are far better conditioned
    for k, (rtol, atol) in enumerate(((3e-3, 2e-7), (2e-2, 1e-12), (1e-4, 2e-8), (1e-3, 1e-12),
                                      (1e-4, 2e-8), (1e-3, 1e-12))):
        np.testing.assert_allclose(got[:, :, k], want[:, :, k], rtol=rtol, atol=atol * w * h)


def test_chain_identical_inputs_give_zeros():
    ref, _ = _xyb_like(3, 31, 22)
    got = oracle.ss2_chain(ref, ref, 6, oracle.ss2_cascade_coefficients(1.5))
    assert np.all(got == 0.0)


def test_chain_later_scale_is_the_first_scale_of_the_downsampled_planes():
    ref, dis = _xyb_like(5, 27, 18, nch=2)
    coef = oracle.ss2_cascade_coefficients(1.5)
    full = oracle.ss2_chain(ref, dis, 3, coef)
    r2 = [oracle.ss2_downsample(oracle.ss2_downsample(p)) for p in ref]
    d2 = [oracle.ss2_downsample(oracle.ss2_downsample(p)) for p in dis]
    assert np.array_equal(full[2], oracle.ss2_chain(r2, d2, 1, coef)[0])
    assert np.array_equal(full[0], oracle.ss2_chain(ref, dis, 1, coef)[0])


def test_chain_first_scale_is_the_statistics_of_the_blurred_planes():
    ref, dis = _xyb_like(6, 21, 14, nch=1)
    coef = oracle.ss2_cascade_coefficients(1.5)
    a, b = ref[0], dis[0]
    blurred = [oracle.ss2_blur(p, coef) for p in (a, b, a * a, b * b, a * b)]
    want = oracle.ss2_channel_sums(a, b, *blurred)
    assert np.array_equal(oracle.ss2_chain(ref, dis, 1, coef)[0, 0], want)


def test_chain_refuses_bad_arguments():
    ref, dis = _xyb_like(8, 8, 8, nch=1)
    coef = oracle.ss2_cascade_coefficients(1.5)
    for ns in (0, 7):
        with pytest.raises(oracle.OracleError):
            oracle.ss2_chain(ref, dis, ns, coef)
