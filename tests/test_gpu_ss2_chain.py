"""The device's ssimulacra2 per-scale chain against the oracle, on an MI355X.

"Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
SYCL", Findings 2 and 7.  Bars:
  * the blur (both passes) and the downsample equal the oracle's bit for bit
    (Finding 2: everything but the sums reproduces the CPU exactly);
  * the six sums per channel and scale lie within 1e-10 relative of the
    oracle's fp64 sequential sums, plus 2^-45 per pixel for the rounding of
    each term's quotient (the blurred planes are identical, so only the terms'
    last bits and the order of the sums differ), and are bitwise repeatable;
  * identical inputs give zeros at every scale.
Every call goes through the C ABI.
"""

import sys

import numpy as np
import pytest

import oracle
from full_reference_video_amd import synth, vqm

pytestmark = pytest.mark.gpu

REL = 1e-10
# Distinct dyadic coefficients of both signs, and a stable set with complex
# poles: the recursion's wiring is visible in every output bit.
DYADIC = np.array([0.5, 0.25, -0.125, 0.0625], np.float32)
COMPLEX = np.array([0.136, 1.6, -0.94, 0.204], np.float32)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _bits_equal(got, want):
    got = np.ascontiguousarray(got, np.float32)
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad[0].size == 0, (len(bad[0]), [b[:5] for b in bad], got[bad][:5], want[bad][:5])


@pytest.mark.parametrize("sigma", [0.5, 1.5, 2.0, 7.25])
def test_cascade_coefficients_match_the_oracle(torch_cuda, sigma):
    _bits_equal(vqm.vqm_ss2_cascade_coefficients(sigma), oracle.ss2_cascade_coefficients(sigma))


COEFS = {"cascade1.5": None, "complex": COMPLEX, "dyadic": DYADIC}


def _coef(name):
    return oracle.ss2_cascade_coefficients(1.5) if name == "cascade1.5" else COEFS[name]


@pytest.mark.parametrize("coef", sorted(COEFS))
@pytest.mark.parametrize("h,w", [(1, 1), (1, 33), (33, 1), (64, 32), (65, 33), (97, 130), (128, 31),
                                 (324, 576), (481, 853), (2160, 3840)])
def test_blur_bit_exact(torch_cuda, coef, h, w):
    c = _coef(coef)
    rng = np.random.default_rng(h * 7919 + w)
    plane = rng.uniform(0.0, 1.0, (h, w)).astype(np.float32)
    say(f"blur {w}x{h} {coef}")
    want = oracle.ss2_blur(plane, c)
    got = vqm.vqm_ss2_blur(_dev(torch_cuda, plane), c).cpu().numpy()
    _bits_equal(got, want)


def test_blur_in_place(torch_cuda):
    c = _coef("cascade1.5")
    plane = np.random.default_rng(3).uniform(0.0, 1.0, (77, 141)).astype(np.float32)
    t = _dev(torch_cuda, plane)
    vqm.vqm_ss2_blur(t, c, out=t)
    _bits_equal(t.cpu().numpy(), oracle.ss2_blur(plane, c))


def test_blur_of_an_impulse_keeps_its_subnormal_tail(torch_cuda):
    # The response decays geometrically through fp32's subnormal range along
    # the row; the device must carry it as the CPU does (no flush to zero).
    c = _coef("cascade1.5")
    plane = np.zeros((3, 300), np.float32)
    plane[1, 2] = 1.0
    want = oracle.ss2_blur(plane, c)
    assert np.any((want != 0) & (np.abs(want) < np.finfo(np.float32).tiny))
    _bits_equal(vqm.vqm_ss2_blur(_dev(torch_cuda, plane), c).cpu().numpy(), want)


@pytest.mark.parametrize("h,w", [(1, 1), (2, 3), (5, 7), (8, 8), (481, 853), (2160, 3840)])
def test_downsample_bit_exact(torch_cuda, h, w):
    plane = np.random.default_rng(h + w).uniform(0.0, 1.0, (h, w)).astype(np.float32)
    _bits_equal(vqm.vqm_ss2_downsample(_dev(torch_cuda, plane)).cpu().numpy(), oracle.ss2_downsample(plane))


def _check_close(got, want, npix):
    # Beside the relative bar, each pixel's term may differ by its two
    # quotients' rounding: the oracle's fp64 division (2^-53 relative) and the
    # device's ff_div (about 2^-46), both below 2^-45 absolute for terms formed
    # from quotients near 1.  That matters only where a sum is tiny, as on the
    # last scales of small planes, where 1 - q cancels.
    for idx in np.ndindex(want.shape):
        tol = REL * abs(want[idx]) + npix * 2.0 ** -45
        assert abs(got[idx] - want[idx]) <= tol, (idx, got[idx], want[idx])


@pytest.mark.parametrize("w,h,nch,nscales", [(576, 324, 3, 6), (853, 481, 3, 6), (1920, 1080, 1, 4),
                                             (17, 9, 2, 6), (1, 1, 1, 1), (3, 2, 3, 6), (3840, 2160, 3, 6)])
def test_scale_sums_match_the_oracle(torch_cuda, w, h, nch, nscales):
    torch = torch_cuda
    ref, dis = synth.ss2_images(11, w, h, nch)
    coef = oracle.ss2_cascade_coefficients(1.5)
    say(f"chain {w}x{h}, {nch} channels, {nscales} scales")
    want = oracle.ss2_chain(ref, dis, nscales, coef)
    dr, dd = [_dev(torch, p) for p in ref], [_dev(torch, p) for p in dis]
    got = vqm.vqm_ss2_scale_sums(dr, dd, nscales, coef)
    worst = np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-300))
    say(f"  largest relative difference {worst:.3e}")
    _check_close(got, want, w * h)
    assert np.array_equal(vqm.vqm_ss2_scale_sums(dr, dd, nscales, coef), got)


def test_scale_sums_of_identical_inputs_are_zero(torch_cuda):
    ref, _ = synth.ss2_images(12, 300, 170, 3)
    dr = [_dev(torch_cuda, p) for p in ref]
    got = vqm.vqm_ss2_scale_sums(dr, dr, 6, oracle.ss2_cascade_coefficients(1.5))
    assert np.all(got == 0.0)


def test_scale_sums_after_a_larger_frame(torch_cuda):
    # The workspace grows for a large frame and is reused for a small one.
    coef = oracle.ss2_cascade_coefficients(1.5)
    for w, h in ((1280, 720), (96, 64)):
        ref, dis = synth.ss2_images(13, w, h, 2)
        want = oracle.ss2_chain(ref, dis, 5, coef)
        got = vqm.vqm_ss2_scale_sums([_dev(torch_cuda, p) for p in ref], [_dev(torch_cuda, p) for p in dis], 5,
                                     coef)
        _check_close(got, want, w * h)


def test_chain_refuses_bad_arguments(torch_cuda):
    ref, dis = synth.ss2_images(14, 32, 16, 1)
    coef = oracle.ss2_cascade_coefficients(1.5)
    with pytest.raises(TypeError):
        vqm.vqm_ss2_scale_sums(ref, dis, 2, coef)  # numpy arrays, not device tensors
    dr, dd = [_dev(torch_cuda, p) for p in ref], [_dev(torch_cuda, p) for p in dis]
    for ns in (0, 7):
        with pytest.raises(vqm.VqmError):
            vqm.vqm_ss2_scale_sums(dr, dd, ns, coef)
    with pytest.raises(vqm.VqmError):
        vqm.vqm_ss2_scale_sums(dr, dd, 2, np.array([np.nan, 0, 0, 0], np.float32))
    with pytest.raises(vqm.VqmError):
        vqm.vqm_ss2_scale_sums(dr * 4, dd * 4, 2, coef)  # four channels


@pytest.mark.parametrize("w,h,nch,nscales", [(576, 324, 3, 6), (130, 117, 2, 6), (97, 45, 1, 1), (64, 51, 1, 3),
                                             (33, 2, 2, 6), (1, 1, 1, 6), (129, 65, 1, 6), (3840, 2160, 1, 6),
                                             (1031, 777, 3, 6)])
def test_chain_kernels_blur_bit_exact(torch_cuda, w, h, nch, nscales):
    # The chain's own pyramid and five-plane row and column kernels (not the
    # one-plane blur's or downsample's): every blurred plane of every scale
    # equal bit for bit to the oracle's blur of the oracle's downsampled
    # images, and the sums of the same launch within the bar.
    ref, dis = synth.ss2_images(15, w, h, nch)
    coef = oracle.ss2_cascade_coefficients(1.5)
    say(f"chain kernels' blurred planes {w}x{h}, {nch} channels, {nscales} scales")
    sums, planes = vqm.vqm_debug_ss2_blurred([_dev(torch_cuda, p) for p in ref], [_dev(torch_cuda, p) for p in dis],
                                             coef, nscales)
    a_s, b_s = list(ref), list(dis)
    for s in range(nscales):
        got = planes[s].cpu().numpy()
        for c in range(nch):
            a, b = a_s[c], b_s[c]
            for k, src in enumerate((a, b, a * a, b * b, a * b)):
                _bits_equal(got[c, k], oracle.ss2_blur(src, coef))
        a_s = [oracle.ss2_downsample(p) for p in a_s]
        b_s = [oracle.ss2_downsample(p) for p in b_s]
    _check_close(sums, oracle.ss2_chain(ref, dis, nscales, coef), w * h)


def test_submitted_frames_equal_the_blocking_call(torch_cuda):
    # Frames of different sizes, channel and scale counts in flight together
    # on one context, each on its own slot stream: collected in submission
    # order, each equal bit for bit to the blocking call and within the bar
    # of the oracle; a fourth frame is refused while three are in flight.
    torch = torch_cuda
    coef = oracle.ss2_cascade_coefficients(1.5)
    cases = [(576, 324, 3, 6), (130, 97, 2, 4), (1920, 1080, 1, 5), (33, 17, 3, 6), (853, 481, 3, 6)]
    frames = []
    for k, (w, h, nch, ns) in enumerate(cases):
        ref, dis = synth.ss2_images(20 + k, w, h, nch)
        frames.append((ref, dis, [_dev(torch, p) for p in ref], [_dev(torch, p) for p in dis], ns))
    with vqm.Context(0) as ctx:
        with pytest.raises(vqm.VqmError):
            ctx.vqm_ss2_collect()  # nothing in flight
        got = []
        for k, (_, _, dr, dd, ns) in enumerate(frames):
            if ctx.vqm_ss2_in_flight() == vqm.VQM_SS2_MAX_IN_FLIGHT:
                with pytest.raises(vqm.VqmError):
                    ctx.vqm_ss2_submit(dr, dd, ns, coef)
                got.append(ctx.vqm_ss2_collect())
            say(f"submit {cases[k]}")
            ctx.vqm_ss2_submit(dr, dd, ns, coef)
        while ctx.vqm_ss2_in_flight():
            got.append(ctx.vqm_ss2_collect())
    assert len(got) == len(frames)
    for (ref, dis, dr, dd, ns), g, (w, h, _, _) in zip(frames, got, cases):
        assert np.array_equal(g, vqm.vqm_ss2_scale_sums(dr, dd, ns, coef))
        _check_close(g, oracle.ss2_chain(ref, dis, ns, coef), w * h)


def test_submit_orders_after_the_context_stream(torch_cuda):
    # A context on torch's stream: planes written by torch just before the
    # submit are the ones the chain reads (the slot stream waits for the
    # context's stream), and a context closed with frames in flight waits
    # for them.
    torch = torch_cuda
    coef = oracle.ss2_cascade_coefficients(1.5)
    ref, dis = synth.ss2_images(30, 1280, 720, 3)
    src_r = [_dev(torch, p) for p in ref]
    src_d = [_dev(torch, p) for p in dis]
    want = oracle.ss2_chain(ref, dis, 6, coef)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dr = [torch.zeros_like(t) for t in src_r]
        dd = [torch.zeros_like(t) for t in src_d]
        torch.cuda.synchronize()
        ctx = vqm.Context(0, stream=s)
        for a, b in zip(dr + dd, src_r + src_d):
            torch.cuda._sleep(1_000_000)  # the copies land well after the submit returns
            a.copy_(b)
        ctx.vqm_ss2_submit(dr, dd, 6, coef)
        got = ctx.vqm_ss2_collect()
        ctx.vqm_ss2_submit(dr, dd, 6, coef)
        ctx.close()  # one frame still in flight
    _check_close(got, want, 1280 * 720)
    torch.cuda.synchronize()
