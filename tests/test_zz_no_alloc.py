"""The allocation-free float_ssim entry point against the blocking call.

``vqm_ssim_frame_noalloc`` enqueues the float_ssim kernels on a caller's
stream with its scratch in a fixed device array, allocating nothing.  Its
score must equal ``vqm_ssim_frame``'s bit for bit (the same kernels and the
same fixed reduction tree) and lie within 5e-5 of the oracle, on calls in a
row whose frames shrink (the array keeps the last call's contents).
"""

import errno
import sys

import numpy as np
import pytest

import oracle
from full_reference_video_amd import synth, vqm

pytestmark = pytest.mark.gpu

TOL = 5e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(torch, a):
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.cuda()


# (workload, frame, width, height, bpc): 2160p 10-bit (s = 8), then smaller
# frames: 853x481 12-bit (s = 2, odd width), 576x324 8-bit (s = 1, raw map),
# 1280x720 16-bit (s = 3, the general decimation).
CASES = [(4, 0, None, None, None), (2, 5, None, None, None), (1, 0, None, None, None),
         (4, 2, 1280, 720, 16)]


def _frames(c, t, w, h, bpc):
    kw = {k: v for k, v in (("w", w), ("h", h), ("bpc", bpc)) if v is not None}
    src = synth.FrameSource(c, **kw)
    ref, dis = src.pair(t)
    return src, ref, dis


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_noalloc_equals_the_blocking_call_on_shrinking_frames(torch_cuda, where):
    torch = torch_cuda
    if where == "device":
        score = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    else:
        score = torch.full((1,), float("nan"), dtype=torch.float64).pin_memory()
    stream = torch.cuda.Stream()
    for rnd in range(2):
        for c, t, w, h, bpc in CASES:
            src, ref, dis = _frames(c, t, w, h, bpc)
            say(f"noalloc ({where}) round {rnd}: {src.w}x{src.h} bpc {src.bpc}")
            r, d = to_dev(torch, ref), to_dev(torch, dis)
            torch.cuda.synchronize()
            score.fill_(float("nan"))
            torch.cuda.synchronize()
            vqm.vqm_ssim_frame_noalloc(r, d, src.bpc, score, stream)
            stream.synchronize()
            got = float(score.cpu()[0])
            want = vqm.vqm_ssim_frame(r, d, src.bpc)
            assert got == want, (got, want)
            assert abs(got - oracle.ssim(ref, dis, src.bpc)) <= TOL


def test_noalloc_two_calls_in_a_row_on_one_stream(torch_cuda):
    # Two frames back to back on the legacy default stream, the second
    # smaller, into two score slots, then one wait: the second call's kernels
    # run after the first's on the same stream and reuse the same array.
    torch = torch_cuda
    a = _frames(4, 7, None, None, None)
    b = _frames(3, 3, None, None, None)
    scores = torch.full((2,), float("nan"), dtype=torch.float64, device="cuda")
    devs = [(to_dev(torch, x[1]), to_dev(torch, x[2]), x[0].bpc) for x in (a, b)]
    torch.cuda.synchronize()
    say("noalloc: 2160p then 1080p on the default stream")
    for k, (r, d, bpc) in enumerate(devs):
        vqm.vqm_ssim_frame_noalloc(r, d, bpc, scores[k:k + 1], None)
    torch.cuda.synchronize()
    got = scores.cpu().tolist()
    for k, (r, d, bpc) in enumerate(devs):
        assert got[k] == vqm.vqm_ssim_frame(r, d, bpc)


def test_noalloc_refuses_what_it_cannot_take(torch_cuda):
    torch = torch_cuda
    src, ref, dis = _frames(1, 0, None, None, None)
    score = torch.zeros(1, dtype=torch.float64, device="cuda")
    with pytest.raises(vqm.VqmError) as e:
        vqm.vqm_ssim_frame_noalloc(ref, dis, 8, score, None)  # host planes
    assert e.value.rc == -errno.EINVAL
    r, d = to_dev(torch, ref), to_dev(torch, dis)
    with pytest.raises(vqm.VqmError) as e:
        vqm.vqm_ssim_frame_noalloc(r, d, 8, torch.zeros(1, dtype=torch.float64), None)  # pageable score
    assert e.value.rc == -errno.EINVAL
    small = torch.zeros((10, 300), dtype=torch.uint8, device="cuda")
    with pytest.raises(vqm.VqmError) as e:
        vqm.vqm_ssim_frame_noalloc(small, small, 8, score, None)  # below the 11x11 window
    assert e.value.rc == -errno.ENOTSUP
    torch.cuda.synchronize()
