"""The device's ssimulacra2 per-scale statistics against the oracle, on an MI355X.

"Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
SYCL", Findings 3-5.  Bars:
  * the fp32-pair operations (every step correctly rounded) equal the
    oracle's bit for bit;
  * the six sums per channel lie within 1e-10 relative of the oracle's fp64
    sequential sums (the oracle's own rounding bound at a 3840x2160 plane is
    n * 2^-53 ~ 9e-10 relative; the pair terms carry ~2^-46), and are bitwise
    repeatable whatever the planes' alignment;
  * identical inputs give six exact zeros.
Every call goes through the C ABI.
"""

import sys

import numpy as np
import pytest

import oracle
from full_reference_video_amd import synth, vqm

pytestmark = pytest.mark.gpu

REL = 1e-10


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _rand_pairs(rng, n, lo_exp=-20, hi_exp=20):
    """Normalised pairs: hi of random sign and magnitude 2^lo_exp..2^hi_exp,
    lo below half an ulp of hi."""
    mag = np.exp2(rng.uniform(lo_exp, hi_exp, n)) * rng.choice([-1.0, 1.0], n)
    hi = mag.astype(np.float32)
    lo = (np.spacing(np.abs(hi)).astype(np.float64) * rng.uniform(-0.5, 0.5, n)).astype(np.float32)
    return np.stack([hi, lo], axis=1)


@pytest.mark.parametrize("op,name", [(0, "two_sum"), (1, "two_prod"), (2, "ff_add"), (3, "ff_mul"), (4, "ff_div")])
def test_pair_ops_bit_exact(torch_cuda, op, name):
    rng = np.random.default_rng(100 + op)
    n = 6000
    a, b = _rand_pairs(rng, n), _rand_pairs(rng, n)
    # a few structured cases: equal and opposite operands, exact ratios
    a[:4] = [[1.0, 0.0], [3.0, 0.0], [0.1, 0.0], [-2.5, 0.0]]
    b[:4] = [[1.0, 0.0], [-3.0, 0.0], [0.3, 0.0], [0.5, 0.0]]
    say(f"pair op {name} on {n} pairs")
    got = vqm.vqm_debug_pair_ops(op, a, b)
    fn = {0: lambda x, y: oracle.two_sum(x[0], y[0]), 1: lambda x, y: oracle.two_prod(x[0], y[0]),
          2: oracle.ff_add, 3: oracle.ff_mul, 4: oracle.ff_div}[op]
    want = np.array([fn(a[i], b[i]) for i in range(n)], np.float32)
    bad = np.nonzero(np.any(got.view(np.uint32) != want.view(np.uint32), axis=1))[0]
    assert bad.size == 0, (name, bad[:5], got[bad[:5]], want[bad[:5]])


def _dev(torch, channels, offset=0):
    """Device copies of the planes; offset > 0 puts each plane `offset`
    floats into its allocation (breaking 16-byte alignment)."""
    out, keep = [], []
    for planes in channels:
        row = []
        for p in planes:
            h, w = p.shape
            buf = torch.empty(h * w + offset, dtype=torch.float32, device="cuda")
            t = buf[offset:].view(h, w)
            t.copy_(torch.from_numpy(p))
            row.append(t)
            keep.append(buf)
        out.append(row)
    return out, keep


def _check_close(got, want, n):
    for c in range(want.shape[0]):
        for k in range(6):
            tol = REL * abs(want[c, k]) + n * 2.0 ** -100
            assert abs(got[c, k] - want[c, k]) <= tol, (c, k, got[c, k], want[c, k])


@pytest.mark.parametrize("w,h,nch", [(576, 324, 3), (853, 481, 3), (3840, 2160, 3), (1920, 1080, 1),
                                     (1, 1, 1), (7, 3, 2), (5, 1, 3), (1023, 17, 1)])
def test_ss2_sums_match_the_oracle(torch_cuda, w, h, nch):
    torch = torch_cuda
    channels = synth.ss2_planes(3, w, h, nch)
    say(f"ss2 sums {w}x{h}, {nch} channels")
    want = np.array([oracle.ss2_channel_sums(*c) for c in channels])
    dev, _keep = _dev(torch, channels)
    torch.cuda.synchronize()
    got = vqm.vqm_ss2_channel_sums(dev)
    worst = np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-300))
    say(f"  largest relative difference {worst:.3e}")
    _check_close(got, want, w * h)
    # repeatable, and the same bits when the planes are not 16-byte aligned
    assert np.array_equal(vqm.vqm_ss2_channel_sums(dev), got)
    dev2, _keep2 = _dev(torch, channels, offset=1)
    torch.cuda.synchronize()
    assert np.array_equal(vqm.vqm_ss2_channel_sums(dev2), got)


def test_ss2_identical_inputs_give_zeros(torch_cuda):
    torch = torch_cuda
    channels = synth.ss2_planes(4, 640, 360, 3)
    same = [[c[0], c[0], c[2], c[2], c[4], c[4], c[4]] for c in channels]
    dev, _keep = _dev(torch, same)
    torch.cuda.synchronize()
    got = vqm.vqm_ss2_channel_sums(dev)
    assert np.all(got == 0.0)
    want = np.array([oracle.ss2_channel_sums(*c) for c in same])
    assert np.all(want == 0.0)


def test_ss2_constant_planes(torch_cuda):
    torch = torch_cuda
    h, w = 37, 53
    mk = lambda v: np.full((h, w), v, np.float32)
    a, b = 0.25, 0.5
    channels = [[mk(a), mk(b), mk(a), mk(b), mk(a * a), mk(b * b), mk(a * b)]]
    dev, _keep = _dev(torch, channels)
    torch.cuda.synchronize()
    got = vqm.vqm_ss2_channel_sums(dev)[0]
    d = (a - b) ** 2
    assert got[0] == pytest.approx(h * w * d, rel=1e-13)
    assert got[1] == pytest.approx(h * w * d ** 4, rel=1e-12)
    assert np.all(got[2:] == 0.0)


def test_ss2_refuses_host_planes_and_bad_counts(torch_cuda):
    channels = synth.ss2_planes(5, 32, 16, 1)
    with pytest.raises(TypeError):
        vqm.vqm_ss2_channel_sums(channels)  # numpy arrays, not device tensors
    dev, _keep = _dev(torch_cuda, channels * 4)
    with pytest.raises(vqm.VqmError):
        vqm.vqm_ss2_channel_sums(dev)       # four channels
