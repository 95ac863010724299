"""Pins of the oracle's ssimulacra2 statistics and pair arithmetic.

"Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
SYCL", Findings 3-4.  Each check holds the oracle against something other than
itself: exact rational arithmetic (Python ``Fraction``), invariants and closed
forms.  The rational check rounds the definition's three fp32 quantities with
numpy float32 arithmetic and evaluates the fp64 terms and the sums exactly.
"""

from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle

U = Fraction(1, 1 << 24)  # fp32 unit roundoff
C2 = Fraction(np.float32(0.0009).item())


def F(x):
    return Fraction(float(x))


def pair_value(p):
    return F(p[0]) + F(p[1])


# ---------------------------------------------------------------- pairs

finite32 = st.floats(min_value=-2.0 ** 60, max_value=2.0 ** 60, allow_nan=False, allow_infinity=False, width=32)
normal32 = finite32.filter(lambda x: x == 0.0 or abs(x) > 1e-15)
pos32 = st.floats(min_value=2.0 ** -20, max_value=2.0 ** 20, allow_nan=False, allow_infinity=False, width=32)


@settings(max_examples=400, deadline=None)
@given(finite32, finite32)
def test_two_sum_is_exact(a, b):
    s, e = oracle.two_sum(a, b)
    assert s == np.float32(np.float32(a) + np.float32(b))
    assert F(s) + F(e) == F(a) + F(b)


@settings(max_examples=400, deadline=None)
@given(normal32, normal32)
def test_two_prod_is_exact(a, b):
    if a != 0.0 and b != 0.0 and abs(a * b) < 1e-20:
        return  # the error term would underflow
    p, e = oracle.two_prod(a, b)
    assert p == np.float32(np.float32(a) * np.float32(b))
    assert F(p) + F(e) == F(a) * F(b)


def _pair(hi, frac):
    """A normalised pair: hi and a low part below half an ulp of hi."""
    hi = np.float32(hi)
    lo = np.float32(float(np.spacing(hi)) * 0.5 * frac)
    return np.array([hi, lo], np.float32)


pairs = st.tuples(pos32, st.floats(min_value=-0.999, max_value=0.999), st.sampled_from([1, -1])).map(
    lambda t: _pair(t[0] * t[2], t[1]))


@settings(max_examples=400, deadline=None)
@given(pairs, pairs)
def test_ff_add_error_bound(a, b):
    got = pair_value(oracle.ff_add(a, b))
    exact = pair_value(a) + pair_value(b)
    assert abs(got - exact) <= 3 * U * U * abs(exact) + Fraction(1, 1 << 149)


@settings(max_examples=400, deadline=None)
@given(pairs, pairs)
def test_ff_mul_error_bound(a, b):
    got = pair_value(oracle.ff_mul(a, b))
    exact = pair_value(a) * pair_value(b)
    assert abs(got - exact) <= 7 * U * U * abs(exact)


@settings(max_examples=600, deadline=None)
@given(pairs, pairs)
def test_ff_div_error_bound(a, b):
    got = pair_value(oracle.ff_div(a, b))
    exact = pair_value(a) / pair_value(b)
    # the page's figure: relative error about 2^-46 (16 u^2 = 2^-44 as a bound)
    assert abs(got - exact) <= 16 * U * U * abs(exact)


def test_ff_div_beats_one_fp32_quotient():
    # Where one correctly rounded quotient errs by ~2^-25, the pair is far
    # closer: 1/3, 2/7, 10/9 ...
    for n, d in [(1, 3), (2, 7), (10, 9), (123456, 7), (1, 1.1)]:
        got = pair_value(oracle.ff_div((n, 0.0), (d, 0.0)))
        exact = F(np.float32(n)) / F(np.float32(d))
        single = F(np.float32(np.float32(n) / np.float32(d)))
        assert abs(got - exact) < abs(single - exact) * Fraction(1, 1 << 18)


# ---------------------------------------------------------------- the six sums

def _exact_planes(rng, h, w):
    """Seven planes on coarse binary grids (means and images on 2^-6 in
    [0, 1), second moments on 2^-12 near the squares of the means), so that
    the image differences are exact and only the steps that add C2 round."""
    g6 = lambda shape: rng.integers(0, 64, size=shape).astype(np.float32) / 64
    mu1, mu2 = g6((h, w)), g6((h, w))
    img1 = np.clip(mu1 + (rng.integers(-8, 9, size=(h, w)) / 64).astype(np.float32), 0, 1).astype(np.float32)
    img2 = np.clip(mu2 + (rng.integers(-8, 9, size=(h, w)) / 64).astype(np.float32), 0, 1).astype(np.float32)
    var = lambda: (rng.integers(0, 40, size=(h, w)) / 4096).astype(np.float32)
    s11 = (mu1 * mu1 + var()).astype(np.float32)
    s22 = (mu2 * mu2 + var()).astype(np.float32)
    s12 = (mu1 * mu2 + (rng.integers(-30, 40, size=(h, w)) / 4096).astype(np.float32)).astype(np.float32)
    return img1, img2, mu1, mu2, s11, s22, s12


def _f32(x):
    return np.float32(x)


def _exact_sums(img1, img2, mu1, mu2, s11, s22, s12):
    """The definition with its fp32 steps rounded once each by numpy's
    float32 arithmetic (IEEE round-to-nearest per operation) and everything
    after them, the fp64 terms and the sums, in exact rationals."""
    acc = [Fraction(0)] * 6
    c2 = _f32(0.0009)
    for i in np.ndindex(mu1.shape):
        m1, m2 = _f32(mu1[i]), _f32(mu2[i])
        dm = _f32(m1 - m2)
        num_m = F(_f32(_f32(1.0) - _f32(dm * dm)))
        num_s = F(_f32(_f32(_f32(2.0) * _f32(s12[i] - _f32(m1 * m2))) + c2))
        den_s = F(_f32(_f32(_f32(s11[i] - _f32(m1 * m1)) + _f32(s22[i] - _f32(m2 * m2))) + c2))
        m1, m2 = F(m1), F(m2)
        d = max(1 - num_m * num_s / den_s, Fraction(0))
        e = (1 + abs(F(img2[i]) - m2)) / (1 + abs(F(img1[i]) - m1)) - 1
        art, det = max(e, Fraction(0)), max(-e, Fraction(0))
        for k, v in enumerate((d, d ** 4, art, art ** 4, det, det ** 4)):
            acc[k] += v
    return acc


@pytest.mark.parametrize("seed,h,w", [(1, 5, 7), (2, 9, 4), (3, 12, 12), (4, 1, 31)])
def test_ss2_sums_equal_exact_rationals(seed, h, w):
    rng = np.random.default_rng(seed)
    planes = _exact_planes(rng, h, w)
    got = oracle.ss2_channel_sums(*planes)
    want = _exact_sums(*planes)
    n = h * w
    for k in range(6):
        # per term a few fp64 roundings, plus n sequential additions
        assert abs(F(got[k]) - want[k]) <= Fraction(2 * n + 8, 1 << 52) * max(abs(want[k]), Fraction(1, 1 << 200)), k
    assert any(v > 0 for v in want[2:4]) and any(v > 0 for v in want[4:6])


def test_ss2_identical_inputs_give_six_zeros():
    rng = np.random.default_rng(7)
    img = rng.random((40, 50), dtype=np.float32)
    mu = rng.random((40, 50), dtype=np.float32)
    s = (mu * mu + rng.random((40, 50), dtype=np.float32) * 0.01).astype(np.float32)
    sums = oracle.ss2_channel_sums(img, img, mu, mu, s, s, s)
    assert np.all(sums == 0.0)


@pytest.mark.parametrize("a,b", [(0.25, 0.5), (0.75, 0.0), (0.5, 0.5)])
def test_ss2_constant_planes_closed_form(a, b):
    # Flat images: every blurred product is the product of the means, so
    # num_s = denom_s = C2, d = (a - b)^2 and the edge terms vanish.
    h, w = 6, 9
    mk = lambda v: np.full((h, w), v, np.float32)
    sums = oracle.ss2_channel_sums(mk(a), mk(b), mk(a), mk(b), mk(a * a), mk(b * b), mk(a * b))
    d = (a - b) ** 2
    assert sums[0] == pytest.approx(h * w * d, rel=1e-15, abs=0)
    assert sums[1] == pytest.approx(h * w * d ** 4, rel=1e-15, abs=0)
    assert np.all(sums[2:] == 0.0)


def test_ss2_edge_ratio_closed_form():
    # One pixel with |r2 - mu2| = 1/2 and |r1 - mu1| = 0: e = 1/2 exactly
    # (an artifact); swapping the images gives (1)/(3/2) - 1 = -1/3 (detail).
    one = lambda v: np.full((1, 1), v, np.float32)
    planes = [one(0.5), one(1.0), one(0.5), one(0.5), one(0.25), one(0.25), one(0.25)]
    s = oracle.ss2_channel_sums(*planes)
    assert s[2] == 0.5 and s[3] == 0.0625 and s[4] == 0.0 and s[5] == 0.0
    planes[0], planes[1] = planes[1], planes[0]
    s = oracle.ss2_channel_sums(*planes)
    assert s[2] == 0.0 and s[4] == pytest.approx(1 / 3, rel=1e-15) and s[5] == pytest.approx(1 / 81, rel=1e-15)


def test_ss2_deficit_is_clamped_at_zero():
    # num_s > denom_s (structure above the variances) makes 1 - q negative:
    # the term and its fourth power count as zero.
    one = lambda v: np.full((1, 1), v, np.float32)
    s = oracle.ss2_channel_sums(one(0.5), one(0.5), one(0.5), one(0.5), one(0.25), one(0.25), one(0.3))
    assert s[0] == 0.0 and s[1] == 0.0


def test_ss2_rejects_bad_arguments():
    import ctypes
    import errno
    z = np.zeros((2, 2), np.float32)
    out = np.zeros(6)
    ptrs = [oracle._ptr(z)] * 7
    L = oracle.lib()
    assert L.vqm_oracle_ss2_channel_sums(None, *ptrs[1:], 2, 2, oracle._ptr(out)) == -errno.EINVAL
    assert L.vqm_oracle_ss2_channel_sums(*ptrs, 0, 2, oracle._ptr(out)) == -errno.EINVAL
    assert L.vqm_oracle_ss2_channel_sums(*ptrs, 2, 2, None) == -errno.EINVAL
    with pytest.raises(ValueError):
        oracle.ss2_channel_sums(z, z, z, z, z, z, np.zeros((2, 3), np.float32))
