"""Parity of the HIP path with the oracle, on an MI355X.

Bars: decimated planes and MS-SSIM pyramid planes bit-exact; every per-frame
score within 5e-5 of the oracle ("ADR-1405: float_ssim_hip decimates on the
device, bit-identical to the CPU", Context); scores bitwise repeatable.
Every call goes through the C ABI (``full_reference_video_amd.vqm``).
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


@pytest.fixture(scope="module")
def ctx(torch_cuda):
    c = vqm.Context(0)
    yield c
    c.close()


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def to_dev(torch, a):
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.cuda()


# ------------------------------------------------------------ decimation

@pytest.mark.parametrize("c", [2, 3, 4])
def test_decimate_bit_exact_on_workload_frames(ctx, c):
    src = synth.FrameSource(c)
    s = oracle.scale(src.w, src.h)
    for t in (0, 1, src.workload.frames - 1):
        ref, dis = src.pair(t)
        say(f"decimate config {c} frame {t} {src.w}x{src.h} bpc {src.bpc} s {s}")
        gr, gd = ctx.vqm_debug_decimate(ref, dis, src.bpc)
        assert np.array_equal(bits(gr), bits(oracle.decimate(ref, src.bpc, s)))
        assert np.array_equal(bits(gd), bits(oracle.decimate(dis, src.bpc, s)))


SCALES = list(range(1, 17)) + [31, 64, 127, 128]


@pytest.mark.parametrize("s", SCALES)
def test_decimate_bit_exact_forced_scale(ctx, s):
    # Fast-path friendly widths (multiples of 16 samples, bottom rows that
    # mirror) and odd sizes (the general kernel), every depth.
    sizes = [(max(16, s) * 12, s * 12 + 1), (s * 11 + 3, s * 11 + 5)]
    for bpc in (8, 9, 10, 11, 12, 16):
        for (w, h) in sizes:
            ref = synth.random_planes(s * 1000 + bpc, w, h, bpc)
            dis = synth.random_planes(s * 1000 + bpc + 7, w, h, bpc)
            say(f"decimate s {s} bpc {bpc} {w}x{h}")
            gr, gd = ctx.vqm_debug_decimate(ref, dis, bpc, s)
            assert np.array_equal(bits(gr), bits(oracle.decimate(ref, bpc, s))), (s, bpc, w, h)
            assert np.array_equal(bits(gd), bits(oracle.decimate(dis, bpc, s))), (s, bpc, w, h)


@pytest.mark.parametrize("bpc,s,w,h", [(16, 2, 8320, 30), (8, 2, 16512, 24), (16, 4, 16384, 48),
                                       (8, 8, 2048, 100)])
def test_decimate_wide_rows_span_several_workgroups(ctx, bpc, s, w, h):
    ref = synth.random_planes(w + bpc, w, h, bpc)
    dis = synth.random_planes(w + bpc + 1, w, h, bpc)
    say(f"decimate wide s {s} bpc {bpc} {w}x{h}")
    gr, gd = ctx.vqm_debug_decimate(ref, dis, bpc, s)
    assert np.array_equal(bits(gr), bits(oracle.decimate(ref, bpc, s)))
    assert np.array_equal(bits(gd), bits(oracle.decimate(dis, bpc, s)))


def test_decimate_extreme_values(ctx):
    for bpc in (8, 10, 16):
        for kind in ("max", "zero", "checker"):
            for s in (2, 3, 8):
                w, h = 16 * s * 11, 13 * s
                p = synth.random_planes(0, w, h, bpc, kind)
                say(f"decimate extreme {kind} s {s} bpc {bpc}")
                gr, _ = ctx.vqm_debug_decimate(p, p, bpc, s)
                assert np.array_equal(bits(gr), bits(oracle.decimate(p, bpc, s)))


@pytest.mark.parametrize("bpc,s", [(8, 16), (10, 8), (12, 4), (14, 2), (16, 2), (12, 8)])
def test_decimate_window_sums_at_the_16_bit_limit(ctx, bpc, s):
    # Where bpc + 2 log2(s) <= 16 the scoring path keeps the decimated planes
    # as 16-bit window sums; all-maximum samples put the sum at its largest
    # (s^2 (2^bpc - 1), just below 2^16 at the limit).  16-bit at s = 2 and
    # 12-bit at s = 8 lie past the limit and keep fp32 planes.  Both the fast
    # path (w a multiple of 16) and the general path (odd w) run.
    for w, h in ((16 * s * 9, 7 * s), (16 * s * 9 + 3, 7 * s + 1)):
        p = synth.random_planes(0, w, h, bpc, "max")
        q = synth.random_planes(bpc, w, h, bpc)
        say(f"decimate limit s {s} bpc {bpc} {w}x{h}")
        gr, gd = ctx.vqm_debug_decimate(p, q, bpc, s)
        assert np.array_equal(bits(gr), bits(oracle.decimate(p, bpc, s))), (bpc, s, w, h)
        assert np.array_equal(bits(gd), bits(oracle.decimate(q, bpc, s))), (bpc, s, w, h)
        assert gr.max() == float(s * s * ((1 << bpc) - 1)) / float(s * s << (bpc - 8))


# ------------------------------------------------------------ float_ssim

@pytest.mark.parametrize("c", [1, 2, 3, 4])
def test_ssim_workload_frames_within_tolerance(ctx, c):
    src = synth.FrameSource(c)
    frames = sorted({0, 1, src.workload.frames // 2, src.workload.frames - 1})
    for t in frames:
        ref, dis = src.pair(t)
        say(f"ssim config {c} frame {t}")
        want = oracle.ssim(ref, dis, src.bpc)
        got = vqm.vqm_ssim_frame(ref, dis, src.bpc)
        assert abs(got - want) <= TOL, (c, t, got, want)


@pytest.mark.parametrize("w,h,bpc", [(300, 200, 8), (400, 300, 10), (700, 500, 12), (853, 481, 9),
                                     (1000, 1000, 11), (1283, 767, 16), (1666, 1001, 10),
                                     (2000, 1200, 8), (4000, 2000, 12)])
def test_ssim_ragged_sizes_and_depths(ctx, w, h, bpc):
    src = synth.FrameSource(4, w=w, h=h, bpc=bpc)
    ref, dis = src.pair(5)
    say(f"ssim {w}x{h} bpc {bpc} s {oracle.scale(w, h)}")
    want = oracle.ssim(ref, dis, bpc)
    ctx.vqm_ssim_submit(ref, dis, bpc)
    got = ctx.vqm_collect()
    assert abs(got - want) <= TOL, (w, h, bpc, got, want)


def test_8k_frames(ctx):
    # The largest common frame, 7680x4320 10-bit: scale round(4320/256) = 17,
    # a scale that is not a power of two (the general decimation), and a
    # six-level-deep MS-SSIM pyramid of 33 M samples.
    src = synth.FrameSource(4, w=7680, h=4320, bpc=10)
    ref, dis = src.pair(2)
    s = oracle.scale(7680, 4320)
    assert s == 17
    say("8k decimation")
    gr, gd = ctx.vqm_debug_decimate(ref, dis, 10)
    assert np.array_equal(bits(gr), bits(oracle.decimate(ref, 10, s)))
    assert np.array_equal(bits(gd), bits(oracle.decimate(dis, 10, s)))
    say("8k float_ssim")
    assert abs(vqm.vqm_ssim_frame(ref, dis, 10) - oracle.ssim(ref, dis, 10)) <= TOL
    say("8k MS-SSIM")
    assert abs(vqm.vqm_msssim_frame(ref, dis, 10) - oracle.msssim(ref, dis, 10)) <= TOL


def test_ssim_minimum_plane(ctx):
    # the smallest accepted decimated plane: one map pixel
    for (w, h) in [(11, 11), (11, 40), (40, 11)]:
        src = synth.FrameSource(1, w=w, h=h)
        ref, dis = src.pair(0)
        say(f"ssim minimum {w}x{h}")
        assert abs(vqm.vqm_ssim_frame(ref, dis, 8) - oracle.ssim(ref, dis, 8)) <= TOL


def test_ssim_identity_is_exactly_one(ctx):
    for c in (1, 2, 3, 4):
        src = synth.FrameSource(c)
        ref, _ = src.pair(0)
        say(f"ssim identity config {c}")
        assert vqm.vqm_ssim_frame(ref, ref, src.bpc) == 1.0


@pytest.mark.parametrize("a,b", [(0, 0), (10, 200), (128, 129), (255, 0)])
def test_ssim_constant_planes(ctx, a, b):
    for (w, h, bpc) in [(300, 200, 8), (1920, 1080, 10)]:
        full = (1 << bpc) - 1
        dt = np.uint8 if bpc == 8 else np.uint16
        ref = np.full((h, w), round(a * full / 255), dt)
        dis = np.full((h, w), round(b * full / 255), dt)
        say(f"ssim constant {a} {b} {w}x{h}")
        assert abs(vqm.vqm_ssim_frame(ref, dis, bpc) - oracle.ssim(ref, dis, bpc)) <= TOL


def test_ssim_repeatable_across_pointer_kinds_and_streams(torch_cuda):
    torch = torch_cuda
    src = synth.FrameSource(4)
    ref, dis = src.pair(3)
    say("ssim pointer kinds")
    base = vqm.vqm_ssim_frame(ref, dis, 10)
    pin_r = torch.from_numpy(ref.view(np.int16)).pin_memory()
    pin_d = torch.from_numpy(dis.view(np.int16)).pin_memory()
    dev_r, dev_d = to_dev(torch, ref), to_dev(torch, dis)
    assert vqm.vqm_ssim_frame(pin_r, pin_d, 10) == base
    assert vqm.vqm_ssim_frame(dev_r, dev_d, 10) == base
    assert vqm.vqm_ssim_frame(pin_r, dis, 10) == base       # mixed kinds
    s = torch.cuda.Stream()
    with vqm.Context(0, s) as c:
        for _ in range(3):
            c.vqm_ssim_submit(dev_r, dev_d, 10)
        assert [c.vqm_collect() for _ in range(3)] == [base] * 3
    assert abs(base - oracle.ssim(ref, dis, 10)) <= TOL


def test_ssim_geometry_changes_between_frames(ctx):
    # A context that alternates sizes must rebuild its scratch every time.
    a = synth.FrameSource(2).pair(0)
    b = synth.FrameSource(3).pair(0)
    c = synth.FrameSource(1).pair(0)
    want = [oracle.ssim(*a, 12), oracle.ssim(*b, 8), oracle.ssim(*c, 8)]
    say("ssim sticky geometry")
    got = []
    for _ in range(2):
        ctx.vqm_ssim_submit(*a, 12)
        ctx.vqm_ssim_submit(*b, 8)
        ctx.vqm_ssim_submit(*c, 8)
        got += [ctx.vqm_collect() for _ in range(3)]
    for i, g in enumerate(got):
        assert abs(g - want[i % 3]) <= TOL
    assert got[:3] == got[3:]


def test_pipelined_submit_collect_and_flow_control(ctx):
    src = synth.FrameSource(3, w=640, h=400)
    n = vqm.VQM_MAX_IN_FLIGHT + 2
    pairs = [src.pair(t) for t in range(n)]
    say("ssim pipelined")
    want = [vqm.vqm_ssim_frame(r, d, 8) for (r, d) in pairs]
    for r, d in pairs[:vqm.VQM_MAX_IN_FLIGHT]:
        ctx.vqm_ssim_submit(r, d, 8)
    with pytest.raises(vqm.VqmError) as e:
        ctx.vqm_ssim_submit(*pairs[vqm.VQM_MAX_IN_FLIGHT], 8)
    assert e.value.rc == -errno.EAGAIN
    got = [ctx.vqm_collect()]
    for r, d in pairs[vqm.VQM_MAX_IN_FLIGHT:]:
        ctx.vqm_ssim_submit(r, d, 8)
        got.append(ctx.vqm_collect())
    while ctx.vqm_in_flight():
        got.append(ctx.vqm_collect())
    assert got == want
    with pytest.raises(vqm.VqmError) as e:
        ctx.vqm_collect()
    assert e.value.rc == -errno.EAGAIN


@pytest.mark.parametrize("c", [1, 2, 3, 4])
def test_batched_submit_equals_single_frames(torch_cuda, ctx, c):
    torch = torch_cuda
    src = synth.FrameSource(c)
    n = 11  # the generator draws any frame index, whatever the workload's count
    pairs = [src.pair(t) for t in range(n)]
    say(f"ssim batches config {c}")
    single = [vqm.vqm_ssim_frame(r, d, src.bpc) for r, d in pairs]
    # device-resident frames in batches of 1..VQM_MAX_BATCH (a ragged last batch)
    dev = [(to_dev(torch, r), to_dev(torch, d)) for r, d in pairs]
    for b in (1, 3, 8, vqm.VQM_MAX_BATCH):
        got = []
        for i in range(0, n, b):
            chunk = dev[i:i + b]
            ctx.vqm_ssim_submit_batch([r for r, _ in chunk], [d for _, d in chunk], src.bpc)
            got += [ctx.vqm_collect() for _ in chunk]
        assert got == single, b
    # host frames, mixed with device frames, in one batch
    mixed_r = [pairs[0][0], dev[1][0], pairs[2][0]]
    mixed_d = [dev[0][1], pairs[1][1], pairs[2][1]]
    ctx.vqm_ssim_submit_batch(mixed_r, mixed_d, src.bpc)
    assert [ctx.vqm_collect() for _ in range(3)] == single[:3]
    for t in (0, n - 1):
        assert abs(single[t] - oracle.ssim(*pairs[t], src.bpc)) <= TOL


def test_batch_limits(ctx):
    src = synth.FrameSource(1)
    r, d = src.pair(0)
    with pytest.raises(ValueError):
        ctx.vqm_ssim_submit_batch([r] * (vqm.VQM_MAX_BATCH + 1), [d] * (vqm.VQM_MAX_BATCH + 1), 8)
    for _ in range(vqm.VQM_MAX_IN_FLIGHT // vqm.VQM_MAX_BATCH):
        ctx.vqm_ssim_submit_batch([r] * vqm.VQM_MAX_BATCH, [d] * vqm.VQM_MAX_BATCH, 8)
    with pytest.raises(vqm.VqmError) as e:
        ctx.vqm_ssim_submit_batch([r], [d], 8)
    assert e.value.rc == -errno.EAGAIN
    vals = [ctx.vqm_collect() for _ in range(vqm.VQM_MAX_IN_FLIGHT)]
    assert len(set(vals)) == 1


def test_gate_on_gpu(ctx):
    z = np.zeros((10, 400), np.uint8)
    with pytest.raises(vqm.VqmError) as e:
        vqm.vqm_ssim_frame(z, z, 8)
    assert e.value.rc == -errno.ENOTSUP
    z = np.zeros((170, 400), np.uint8)
    with pytest.raises(vqm.VqmError) as e:
        ctx.vqm_msssim_submit(z, z, 8)
    assert e.value.rc == -errno.ENOTSUP


# ------------------------------------------------------------ MS-SSIM

def test_msssim_workload_frame(ctx):
    src = synth.FrameSource(5)
    ref, dis = src.pair(0)
    say("msssim config 5 frame 0")
    want, want_lcs = oracle.msssim(ref, dis, 8, want_lcs=True)
    got, lcs = vqm.vqm_msssim_frame_lcs(ref, dis, 8)
    assert abs(got - want) <= TOL, (got, want)
    assert np.all(np.abs(lcs - want_lcs) <= TOL)


@pytest.mark.parametrize("w,h,bpc", [(176, 176, 8), (640, 360, 8), (400, 352, 10), (723, 389, 12),
                                     (1001, 703, 16), (1920, 1080, 8)])
def test_msssim_sizes_and_depths(ctx, w, h, bpc):
    src = synth.FrameSource(5, w=w, h=h, bpc=bpc)
    ref, dis = src.pair(1)
    say(f"msssim {w}x{h} bpc {bpc}")
    want, want_lcs = oracle.msssim(ref, dis, bpc, want_lcs=True)
    ctx.vqm_msssim_submit(ref, dis, bpc)
    got, lcs = ctx.vqm_collect(want_lcs=True)
    assert abs(got - want) <= TOL, (got, want)
    assert np.all(np.abs(lcs - want_lcs) <= TOL)


@pytest.mark.parametrize("w,h,bpc", [(640, 360, 8), (723, 389, 12), (1001, 703, 16)])
def test_msssim_pyramid_bit_exact(ctx, w, h, bpc):
    src = synth.FrameSource(5, w=w, h=h, bpc=bpc)
    ref, dis = src.pair(2)
    xr, xd = oracle.sample_plane(ref, bpc), oracle.sample_plane(dis, bpc)
    for level in range(2, 6):
        xr, xd = oracle.downsample(xr), oracle.downsample(xd)
        say(f"pyramid {w}x{h} bpc {bpc} level {level}")
        gr, gd = ctx.vqm_debug_pyramid(ref, dis, bpc, level)
        assert np.array_equal(bits(gr), bits(xr))
        assert np.array_equal(bits(gd), bits(xd))


# Sizes and batches that take the row-streaming level kernel at levels 1-2
# (strips of 128 columns with a ragged last one, down to a single valid
# column at 1931 wide; odd plane sizes; several strip rows); a batch of one
# frame takes the tile kernel.
# The last case is the MS-SSIM workload's own shape and depth, in its launch batch of 32.
# Odd level-1 widths take one load per sample; even ones one load per sample
# pair (1922 x 1082 at 10 bits: 16-bit pairs), whose odd-width levels (961,
# 1921) read a pair's second sample from the plane's padding at the last
# column.
ROWS_CASES = [(2001, 1203, 16), (1921, 1081, 8), (1283, 767, 12), (1931, 1087, 10), (3840, 2160, 8),
              (1922, 1082, 10), (3842, 2160, 8)]


@pytest.mark.parametrize("w,h,bpc", ROWS_CASES)
def test_msssim_pyramid_bit_exact_in_a_full_batch(ctx, w, h, bpc):
    src = synth.FrameSource(5, w=w, h=h, bpc=bpc)
    n = vqm.VQM_MAX_BATCH
    pairs = [src.pair(t) for t in range(n)]
    sample = (0, n // 2, n - 1)
    want = {t: (oracle.sample_plane(pairs[t][0], bpc), oracle.sample_plane(pairs[t][1], bpc)) for t in sample}
    for level in range(2, 6):
        say(f"batched pyramid {w}x{h} bpc {bpc} level {level}")
        gr, gd = ctx.vqm_debug_pyramid_batch([r for r, _ in pairs], [d for _, d in pairs], bpc, level)
        for t in sample:
            xr, xd = oracle.downsample(want[t][0]), oracle.downsample(want[t][1])
            want[t] = (xr, xd)
            assert np.array_equal(bits(gr[t]), bits(xr)), (level, t)
            assert np.array_equal(bits(gd[t]), bits(xd)), (level, t)


@pytest.mark.parametrize("w,h,bpc", ROWS_CASES)
def test_msssim_score_does_not_depend_on_the_batch(ctx, w, h, bpc):
    # A level's sums are exact (integer terms), so the score is the same
    # bits whichever level kernel the batch size selects.
    src = synth.FrameSource(5, w=w, h=h, bpc=bpc)
    n = vqm.VQM_MAX_BATCH
    pairs = [src.pair(t) for t in range(n)]
    say(f"msssim batch independence {w}x{h} bpc {bpc}")
    ctx.vqm_msssim_submit_batch([r for r, _ in pairs], [d for _, d in pairs], bpc)
    batched = [ctx.vqm_collect(want_lcs=True) for _ in range(n)]
    for t in (0, 7, n - 1):
        s1, l1 = vqm.vqm_msssim_frame_lcs(*pairs[t], bpc)
        assert batched[t][0] == s1, t
        assert np.array_equal(batched[t][1], l1), t
    # batches of 8, 13 and 11 frames take other strip heights (or the tile
    # kernel) at some levels
    say(f"msssim batch independence {w}x{h}: batches of 8, 13, 11")
    i = 0
    for m in (8, 13, 11):
        ctx.vqm_msssim_submit_batch([r for r, _ in pairs[i:i + m]], [d for _, d in pairs[i:i + m]], bpc)
        for t in range(i, i + m):
            got = ctx.vqm_collect(want_lcs=True)
            assert got[0] == batched[t][0], (m, t)
            assert np.array_equal(got[1], batched[t][1]), (m, t)
        i += m
    say(f"msssim batch independence {w}x{h}: oracle")
    assert abs(batched[7][0] - oracle.msssim(*pairs[7], bpc)) <= TOL


def test_msssim_anti_correlated_is_nan(ctx):
    # Inverted planes: the fine levels' mean structure is negative, so the
    # score is NaN (the oracle's pin), alone (tile kernel) and in a full batch
    # (the row kernel at levels 1-2); the level means still match the oracle.
    rng = np.random.default_rng(9)
    ref = rng.integers(0, 256, size=(192, 192)).astype(np.uint8)
    say("msssim anti-correlated 192x192")
    assert np.isnan(vqm.vqm_msssim_frame(ref, 255 - ref, 8))
    ref = rng.integers(0, 256, size=(1081, 1921)).astype(np.uint8)
    dis = (255 - ref).astype(np.uint8)
    n = vqm.VQM_MAX_BATCH
    say("msssim anti-correlated 1921x1081, full batch")
    ctx.vqm_msssim_submit_batch([ref] * n, [dis] * n, 8)
    got = [ctx.vqm_collect(want_lcs=True) for _ in range(n)]
    want, want_lcs = oracle.msssim(ref, dis, 8, want_lcs=True)
    assert np.isnan(want)
    for score, lcs in got:
        assert np.isnan(score)
        assert np.all(np.abs(lcs - want_lcs) <= TOL)
        assert lcs[10] < 0


def test_msssim_identity(ctx):
    src = synth.FrameSource(5, w=960, h=540)
    ref, _ = src.pair(0)
    say("msssim identity")
    score, lcs = vqm.vqm_msssim_frame_lcs(ref, ref, 8)
    assert abs(score - 1.0) <= 1e-6
    assert np.all(lcs[:10] == 1.0)  # luminance and contrast are mirror images


def test_msssim_repeatable(ctx):
    src = synth.FrameSource(5, w=1280, h=720)
    ref, dis = src.pair(4)
    say("msssim repeatable")
    a = vqm.vqm_msssim_frame(ref, dis, 8)
    for _ in range(3):
        ctx.vqm_msssim_submit(ref, dis, 8)
    assert [ctx.vqm_collect() for _ in range(3)] == [a] * 3


def test_msssim_batched_equals_single(ctx):
    src = synth.FrameSource(5, w=960, h=544)
    pairs = [src.pair(t) for t in range(5)]
    say("msssim batch")
    single = [vqm.vqm_msssim_frame_lcs(r, d, 8) for r, d in pairs]
    ctx.vqm_msssim_submit_batch([r for r, _ in pairs], [d for _, d in pairs], 8)
    for s1, l1 in single:
        s2, l2 = ctx.vqm_collect(want_lcs=True)
        assert s2 == s1
        assert np.array_equal(l1, l2)
    assert abs(single[2][0] - oracle.msssim(*pairs[2], 8)) <= TOL


def test_msssim_batches_in_flight_on_both_streams(torch_cuda):
    # A context on a library-owned stream alternates its MS-SSIM batches over
    # that stream and a second one: several batches in flight at once (host
    # and device input, interleaved with float_ssim frames on the first
    # stream), collected in order, give the blocking calls' scores and level
    # means bit for bit; so does a context on a caller's stream, which keeps
    # every batch on that stream.
    torch = torch_cuda
    src = synth.FrameSource(5, w=960, h=544)
    pairs = [src.pair(t) for t in range(12)]
    single = [vqm.vqm_msssim_frame_lcs(r, d, 8) for r, d in pairs]
    ssim_src = synth.FrameSource(2)
    ssim_pair = ssim_src.pair(0)
    ssim_want = vqm.vqm_ssim_frame(*ssim_pair, ssim_src.bpc)
    dev = [(to_dev(torch, r), to_dev(torch, d)) for r, d in pairs]
    torch.cuda.synchronize()
    for stream in (None, torch.cuda.Stream()):
        say(f"msssim batches in flight, stream {stream}")
        with vqm.Context(0, stream) as c:
            for b0 in range(0, 12, 3):
                batch = pairs[b0:b0 + 3] if b0 % 6 == 0 else dev[b0:b0 + 3]
                c.vqm_msssim_submit_batch([r for r, _ in batch], [d for _, d in batch], 8)
                if b0 == 3:
                    c.vqm_ssim_submit(*ssim_pair, ssim_src.bpc)
            got = []
            for k in range(13):
                got.append(c.vqm_collect(want_lcs=True))
        ssim_got = got.pop(6)[0]
        assert ssim_got == ssim_want
        for (s1, l1), (s2, l2) in zip(single, got):
            assert s2 == s1
            assert np.array_equal(l1, l2)


@pytest.mark.parametrize("metric,c", [(0, 2), (0, 4), (1, 5)])
def test_score_frames_loop_matches_single_frames(torch_cuda, metric, c):
    torch = torch_cuda
    src = synth.FrameSource(c, w=960, h=544) if c == 5 else synth.FrameSource(c)
    n = 13
    pairs = [src.pair(t) for t in range(n)]
    say(f"score_frames metric {metric} config {c}")
    one = vqm.vqm_msssim_frame if metric == 1 else vqm.vqm_ssim_frame
    want = [one(r, d, src.bpc) for r, d in pairs]
    dev = [(to_dev(torch, r), to_dev(torch, d)) for r, d in pairs]
    fs = vqm.FrameSet([r for r, _ in dev], [d for _, d in dev], src.bpc)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ctxs = [vqm.Context(0, s) for s in streams]
    try:
        for batch, lag, nc in [(1, 0, 1), (4, 0, 2), (8, 3, 2), (8, 0, 1), (vqm.VQM_MAX_BATCH, 0, 1)]:
            got = vqm.vqm_score_frames(ctxs[:nc], metric, fs, batch, lag)
            assert got.tolist() == want, (batch, lag, nc)
        # host frames through the same loop
        fs_host = vqm.FrameSet([r for r, _ in pairs], [d for _, d in pairs], src.bpc)
        assert vqm.vqm_score_frames(ctxs, metric, fs_host, 5, 0).tolist() == want
    finally:
        for x in ctxs:
            x.close()


def test_mixed_metrics_and_sizes_in_one_context(ctx):
    # float_ssim batches sit in a three-stage pipeline; an MS-SSIM frame or a
    # frame of another size in between must drain it without reordering.
    a = synth.FrameSource(4).pair(1)
    b = synth.FrameSource(5, w=640, h=360).pair(0)
    c = synth.FrameSource(2).pair(3)
    want = [vqm.vqm_ssim_frame(*a, 10), vqm.vqm_msssim_frame(*b, 8), vqm.vqm_ssim_frame(*c, 12)]
    say("mixed metrics pipeline")
    ctx.vqm_ssim_submit_batch([a[0]] * 3, [a[1]] * 3, 10)
    ctx.vqm_msssim_submit(*b, 8)
    ctx.vqm_ssim_submit(*c, 12)
    ctx.vqm_ssim_submit_batch([a[0]] * 2, [a[1]] * 2, 10)
    got = [ctx.vqm_collect() for _ in range(7)]
    assert got == [want[0]] * 3 + [want[1], want[2]] + [want[0]] * 2
    assert abs(want[0] - oracle.ssim(*a, 10)) <= TOL


# ------------------------------------------------------------ full workloads, bench launch shape

def _score_stream(torch, pairs, bpc, metric, batch=vqm.VQM_MAX_BATCH, lag=0, n_streams=1, want_lcs=False,
                  own_streams=True):
    """Score device-resident pairs the way bench.py times them: n_streams
    contexts on library-owned streams (whose MS-SSIM batches alternate over
    two streams each, with the overlapped kernel plans), or with
    own_streams=False on torch streams (every batch on its context's one
    stream), batches of VQM_MAX_BATCH frames per launch, each frame collected
    three batches after its submit (lag 0).  With want_lcs, also the 15
    level means per frame (from a second pass that asks for them)."""
    dev = [(to_dev(torch, r), to_dev(torch, d)) for r, d in pairs]
    fs = vqm.FrameSet([r for r, _ in dev], [d for _, d in dev], bpc)
    ctxs = [vqm.Context(0) if own_streams else vqm.Context(0, torch.cuda.Stream()) for _ in range(n_streams)]
    try:
        first = vqm.vqm_score_frames(ctxs, metric, fs, batch, lag).tolist()
        again = vqm.vqm_score_frames(ctxs, metric, fs, batch, lag).tolist()
        if want_lcs:
            scores, lcs = vqm.vqm_score_frames(ctxs, metric, fs, batch, lag, want_lcs=True)
            assert scores.tolist() == first, "asking for the level means changed a score"
    finally:
        for x in ctxs:
            x.close()
    assert again == first, "scores not bitwise repeatable"
    return (first, lcs) if want_lcs else first


@pytest.mark.parametrize("c", [2, 3, 4])
def test_full_float_ssim_workload_in_bench_launch_shape(torch_cuda, c):
    # Every frame of the workload at its full size, against the oracle frame
    # by frame.
    src = synth.FrameSource(c)
    n = src.workload.frames
    say(f"full workload {c}: generating {n} pairs {src.w}x{src.h} bpc {src.bpc}")
    pairs = [src.pair(t) for t in range(n)]
    say(f"full workload {c}: scoring on the GPU")
    got = _score_stream(torch_cuda, pairs, src.bpc, vqm.VQM_METRIC_FLOAT_SSIM)
    say(f"full workload {c}: oracle")
    worst = 0.0
    for t, (r, d) in enumerate(pairs):
        e = abs(got[t] - oracle.ssim(r, d, src.bpc))
        worst = max(worst, e)
        assert e <= TOL, (c, t, got[t])
    say(f"full workload {c}: worst |gpu - oracle| {worst:.3g}")


def test_full_float_ssim_2160p_two_streams(torch_cuda):
    # The same 2160p frames rotated over two streams give the same bits.
    src = synth.FrameSource(4)
    pairs = [src.pair(t) for t in range(20)]
    say("2160p two streams")
    one = _score_stream(torch_cuda, pairs, src.bpc, vqm.VQM_METRIC_FLOAT_SSIM)
    two = _score_stream(torch_cuda, pairs, src.bpc, vqm.VQM_METRIC_FLOAT_SSIM, n_streams=2)
    assert one == two


def test_full_msssim_workload_in_bench_launch_shape(torch_cuda):
    # All 50 frames scored on the GPU in the bench's launch shape, each score
    # and each of its 15 level means within 5e-5 of the oracle's (stored by
    # tests/golden/make_golden.py, which calls only the oracle: seconds per
    # 2160p frame on one core); one frame is also recomputed by the oracle.
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "msssim_2160p8_oracle.json")) as f:
        rec = json.load(f)["frames"]
    src = synth.FrameSource(5)
    n = src.workload.frames
    say(f"full MS-SSIM workload: generating {n} pairs")
    pairs = [src.pair(t) for t in range(n)]
    say("full MS-SSIM workload: scoring on the GPU")
    got, lcs = _score_stream(torch_cuda, pairs, src.bpc, vqm.VQM_METRIC_MS_SSIM, want_lcs=True)
    single = [vqm.vqm_msssim_frame(r, d, src.bpc) for r, d in pairs]
    assert got == single
    worst = max(abs(got[t] - rec[str(t)]["score"]) for t in range(n))
    worst_lcs = max(float(np.max(np.abs(lcs[t] - np.array(rec[str(t)]["lcs"])))) for t in range(n))
    say(f"full MS-SSIM workload: largest difference from the oracle {worst:.3e} (score), {worst_lcs:.3e} (means)")
    for t in range(n):
        assert abs(got[t] - rec[str(t)]["score"]) <= TOL, (t, got[t], rec[str(t)]["score"])
        assert np.all(np.abs(lcs[t] - np.array(rec[str(t)]["lcs"])) <= TOL), t
    # every batch on one torch stream (the one-stream kernel plans: 136-row
    # level-1 strips where the overlapped batches above took 308), and two
    # contexts of two streams each: the same bits
    say("full MS-SSIM workload: one torch stream")
    assert _score_stream(torch_cuda, pairs, src.bpc, vqm.VQM_METRIC_MS_SSIM, own_streams=False) == single
    say("full MS-SSIM workload: two contexts")
    assert _score_stream(torch_cuda, pairs, src.bpc, vqm.VQM_METRIC_MS_SSIM, n_streams=2) == single
    say("full MS-SSIM workload: oracle frame 23")
    assert abs(got[23] - oracle.msssim(*pairs[23], src.bpc)) <= TOL, got[23]


# ------------------------------------------------------------ enable_db

def _db_bound(s_gpu, s_oracle):
    # The score bar carried through -10 log10(1 - s): its slope is
    # 4.343 / (1 - s), largest at the larger score.
    return 4.35 * TOL / (1.0 - max(s_gpu, s_oracle)) + 1e-9


@pytest.mark.parametrize("c", [1, 2, 3, 4])
def test_ssim_db_form(ctx, c):
    src = synth.FrameSource(c)
    r, d = src.pair(0)
    say(f"dB form config {c}")
    s, db = vqm.vqm_ssim_frame_db(r, d, src.bpc)
    assert s == vqm.vqm_ssim_frame(r, d, src.bpc)
    # the device's log10 against the oracle's, on the same score
    assert abs(db - oracle.db(s)) <= 1e-12 * max(1.0, db)
    so = oracle.ssim(r, d, src.bpc)
    assert abs(db - oracle.db(so)) <= _db_bound(s, so)


def test_ssim_db_identity_and_pipeline(ctx, torch_cuda):
    r, d = synth.FrameSource(2).pair(5)
    s, db = vqm.vqm_ssim_frame_db(r, r, 12)
    assert s == 1.0 and db == float("inf")
    want = vqm.vqm_ssim_frame_db(r, d, 12)
    b = synth.FrameSource(5, w=640, h=360).pair(0)
    ctx.vqm_ssim_submit_batch([r, r], [d, r], 12)
    ctx.vqm_msssim_submit(*b, 8)
    assert ctx.vqm_collect_db() == want
    assert ctx.vqm_collect_db() == (1.0, float("inf"))
    ms, ms_db = ctx.vqm_collect_db()
    assert ms == vqm.vqm_msssim_frame(*b, 8) and np.isnan(ms_db)
    # the scoring loop's dB outputs
    src = synth.FrameSource(3)
    pairs = [src.pair(t) for t in range(11)]
    dev = [(to_dev(torch_cuda, x), to_dev(torch_cuda, y)) for x, y in pairs]
    fs = vqm.FrameSet([x for x, _ in dev], [y for _, y in dev], src.bpc)
    scores, dbs = vqm.vqm_score_frames([ctx], vqm.VQM_METRIC_FLOAT_SSIM, fs, 4, 0, want_db=True)
    for t, (x, y) in enumerate(pairs):
        assert (scores[t], dbs[t]) == vqm.vqm_ssim_frame_db(x, y, src.bpc)


# ------------------------------------------------------------ Y'CbCr pictures

def _yuv_frame(c, t, w, h, bpc, chroma):
    y = synth.FrameSource(c, w=w, h=h, bpc=bpc).pair(t)
    planes = [y]
    for p in (1, 2):
        pw, ph = oracle.plane_dims(w, h, chroma, p)
        planes.append(synth.chroma_pair(c, t, p, pw, ph, bpc))
    return [r for r, _ in planes], [d for _, d in planes]


@pytest.mark.parametrize("w,h,bpc,chroma", [(1920, 1080, 8, 0), (853, 481, 12, 0), (853, 481, 10, 1),
                                            (640, 360, 8, 2), (1921, 1079, 16, 0)])
def test_ssim_yuv_planes(ctx, w, h, bpc, chroma):
    refs, diss = _yuv_frame(3, 2, w, h, bpc, chroma)
    say(f"yuv float_ssim {w}x{h} bpc {bpc} chroma {chroma}")
    scores, db = vqm.vqm_ssim_frame_yuv(refs, diss, bpc, chroma)
    for p in range(3):
        # the same kernels as a lone plane, bit for bit
        assert (scores[p], db[p]) == vqm.vqm_ssim_frame_db(refs[p], diss[p], bpc), p
        assert abs(scores[p] - oracle.ssim(refs[p], diss[p], bpc)) <= TOL, p


@pytest.mark.parametrize("w,h,bpc,chroma", [(1920, 1080, 8, 0), (723, 389, 10, 2)])
def test_msssim_yuv_planes(ctx, w, h, bpc, chroma):
    refs, diss = _yuv_frame(5, 1, w, h, bpc, chroma)
    say(f"yuv MS-SSIM {w}x{h} bpc {bpc} chroma {chroma}")
    scores, lcs = vqm.vqm_msssim_frame_yuv(refs, diss, bpc, chroma)
    for p in range(3):
        one, one_lcs = vqm.vqm_msssim_frame_lcs(refs[p], diss[p], bpc)
        assert scores[p] == one and np.array_equal(lcs[p], one_lcs), p
    # the oracle on the chroma planes (the smaller ones)
    for p in (1, 2):
        assert abs(scores[p] - oracle.msssim(refs[p], diss[p], bpc)) <= TOL, p


def test_yuv_leaves_the_implicit_context_empty(ctx):
    # A refused picture enqueues nothing; the next calls are unaffected.
    w, h = 576, 324
    refs, diss = _yuv_frame(1, 0, w, h, 8, 0)
    with pytest.raises(vqm.VqmError):
        vqm.vqm_msssim_frame_yuv(refs, diss, 8, 0)
    scores, _ = vqm.vqm_ssim_frame_yuv(refs, diss, 8, 0)
    assert scores[0] == vqm.vqm_ssim_frame(refs[0], diss[0], 8)


def test_blocking_calls_from_many_threads(torch_cuda):
    # Blocking calls from threads at once (ctypes releases the GIL around
    # them) each take their own pooled context; threads that come and go
    # reuse the pool.  Every score equals the single-threaded one.
    import threading
    src = synth.FrameSource(2)
    pairs = [src.pair(t) for t in range(5)]
    want = [vqm.vqm_ssim_frame(r, d, 12) for r, d in pairs]
    b = synth.FrameSource(5, w=400, h=352, bpc=10).pair(0)
    want_ms = vqm.vqm_msssim_frame(*b, 10)
    results, errors = {}, []

    def worker(k):
        try:
            got = []
            for _ in range(3):
                got += [vqm.vqm_ssim_frame(r, d, 12) for r, d in pairs]
                got.append(vqm.vqm_msssim_frame(*b, 10))
            results[k] = got
        except Exception as e:  # pragma: no cover - reported below
            errors.append(repr(e))

    say("blocking calls from 6 threads, twice")
    for _ in range(2):
        threads = [threading.Thread(target=worker, args=(k,)) for k in range(6)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
    assert not errors, errors
    for k in range(6):
        assert results[k] == (want + [want_ms]) * 3, k


def _late_default_stream_copy(torch, host):
    """A device tensor whose content arrives late on the default stream.

    It holds zeros at first; a few long fp32 products on the default stream
    (tens of milliseconds) come first, then the copy of ``host`` (pinned), so
    a reader on a stream that does not wait for the default stream sees the
    zeros.
    """
    out = torch.zeros_like(host, device="cuda")
    x = torch.rand(4096, 4096, device="cuda")
    for _ in range(12):
        x = torch.mm(x, x) * (1.0 / 4096)
    out.copy_(host, non_blocking=True)
    return out, x


@pytest.mark.parametrize("metric", ["ssim", "msssim"])
def test_blocking_call_orders_after_default_stream_work(torch_cuda, metric):
    # A plane produced by torch on its default stream, passed straight to a
    # blocking call with no synchronisation: the library's own stream is a
    # blocking stream, so it starts after that work and scores the finished
    # plane.
    torch = torch_cuda
    c = 4 if metric == "ssim" else 5
    src = synth.FrameSource(c, w=960, h=544) if metric == "msssim" else synth.FrameSource(c)
    ref, dis = src.pair(1)
    want = oracle.ssim(ref, dis, src.bpc) if metric == "ssim" else oracle.msssim(ref, dis, src.bpc)
    view = (lambda a: a.view(np.int16)) if src.bpc > 8 else (lambda a: a)
    r = to_dev(torch, ref)
    host = torch.from_numpy(view(dis)).pin_memory()
    torch.cuda.synchronize()
    say(f"{metric}: dis produced on the default stream, scored without a wait")
    for _ in range(2):
        d, keep = _late_default_stream_copy(torch, host)
        fn = vqm.vqm_ssim_frame if metric == "ssim" else vqm.vqm_msssim_frame
        got = fn(r, d, src.bpc)
        assert abs(got - want) <= TOL, (got, want)
    torch.cuda.synchronize()
    # the same through a context on a library-owned stream
    with vqm.Context(0) as cx:
        d, keep = _late_default_stream_copy(torch, host)
        (cx.vqm_ssim_submit if metric == "ssim" else cx.vqm_msssim_submit)(r, d, src.bpc)
        got = cx.vqm_collect()
        assert abs(got - want) <= TOL, (got, want)
    torch.cuda.synchronize()


# ------------------------------------------------------------ recorded passes (graph replay)

def _eager(torch, metric, fs, batch):
    st = torch.cuda.Stream()
    c = vqm.Context(0, st)
    try:
        return vqm.vqm_score_frames([c], metric, fs, batch, 0, want_lcs=metric == vqm.VQM_METRIC_MS_SSIM)
    finally:
        c.close()


def test_graph_replays_match_the_eager_pass(torch_cuda):
    # One recorded float_ssim pass over 40 device frames (a batch of 32 and a
    # ragged one of 8), replayed three times with other GPU work and host
    # waits in between; every replay equals the eager pipelined pass bit for
    # bit.  Then the frames are overwritten in place and the next replay
    # scores the new contents.
    torch = torch_cuda
    src = synth.FrameSource(2)
    n = 40
    pairs = [src.pair(t) for t in range(n)]
    dev = [(to_dev(torch, r), to_dev(torch, d)) for r, d in pairs]
    fs = vqm.FrameSet([r for r, _ in dev], [d for _, d in dev], src.bpc)
    want = _eager(torch, vqm.VQM_METRIC_FLOAT_SSIM, fs, 32)
    for t in (0, n - 1):
        assert abs(want[t] - oracle.ssim(*pairs[t], src.bpc)) <= TOL
    say("graph float_ssim: record")
    with vqm.Graph(0, torch.cuda.Stream(), vqm.VQM_METRIC_FLOAT_SSIM, fs, 32) as g:
        other = synth.FrameSource(4).pair(7)
        for k in range(3):
            say(f"graph float_ssim: replay {k}")
            g.vqm_graph_launch()
            with pytest.raises(vqm.VqmError) as e:
                g.vqm_graph_launch()
            assert e.value.rc == -errno.EBUSY
            got, db = g.vqm_graph_collect(want_db=True)
            assert np.array_equal(got, want), k
            assert np.all(np.isfinite(db))
            with pytest.raises(vqm.VqmError) as e:
                g.vqm_graph_collect()
            assert e.value.rc == -errno.EAGAIN
            vqm.vqm_ssim_frame(*other, 10)                      # eager work in between
            torch.cuda.synchronize()
        # new contents in the same buffers: frames shifted by 40
        new = [src.pair(t) for t in range(n, 2 * n)]
        for (dr, dd), (r, d) in zip(dev, new):
            dr.copy_(to_dev(torch, r))
            dd.copy_(to_dev(torch, d))
        torch.cuda.synchronize()
        want_new = _eager(torch, vqm.VQM_METRIC_FLOAT_SSIM, fs, 32)
        assert not np.array_equal(want_new, want)
        g.vqm_graph_launch()
        assert np.array_equal(g.vqm_graph_collect(), want_new)


def test_graph_msssim_with_level_means(torch_cuda):
    torch = torch_cuda
    src = synth.FrameSource(5, w=960, h=544)
    n = 10
    pairs = [src.pair(t) for t in range(n)]
    dev = [(to_dev(torch, r), to_dev(torch, d)) for r, d in pairs]
    fs = vqm.FrameSet([r for r, _ in dev], [d for _, d in dev], src.bpc)
    want, want_lcs = _eager(torch, vqm.VQM_METRIC_MS_SSIM, fs, 4)
    assert abs(want[3] - oracle.msssim(*pairs[3], src.bpc)) <= TOL
    say("graph MS-SSIM: record and replay twice")
    with vqm.Graph(0, None, vqm.VQM_METRIC_MS_SSIM, fs, 4) as g:
        for _ in range(2):
            g.vqm_graph_launch()
            got, lcs, db = g.vqm_graph_collect(want_lcs=True, want_db=True)
            assert np.array_equal(got, want)
            assert np.array_equal(lcs, want_lcs)
            assert np.all(np.isnan(db))


def test_graph_full_2160p_workload_in_bench_shape(torch_cuda):
    # The 50 frames of the 2160p workload, batches of 32, as bench.py --graph
    # replays them; every frame equals the eager pass, a sample the oracle.
    torch = torch_cuda
    src = synth.FrameSource(4)
    n = src.workload.frames
    say(f"graph 2160p: generating {n} pairs")
    pairs = [src.pair(t) for t in range(n)]
    dev = [(to_dev(torch, r), to_dev(torch, d)) for r, d in pairs]
    fs = vqm.FrameSet([r for r, _ in dev], [d for _, d in dev], src.bpc)
    want = _eager(torch, vqm.VQM_METRIC_FLOAT_SSIM, fs, vqm.VQM_MAX_BATCH)
    with vqm.Graph(0, None, vqm.VQM_METRIC_FLOAT_SSIM, fs, vqm.VQM_MAX_BATCH) as g:
        for k in range(2):
            say(f"graph 2160p: replay {k}")
            g.vqm_graph_launch()
            assert np.array_equal(g.vqm_graph_collect(), want)
    for t in (0, n - 1):
        assert abs(want[t] - oracle.ssim(*pairs[t], src.bpc)) <= TOL


def test_graph_takes_device_frames_only(torch_cuda):
    src = synth.FrameSource(2)
    r, d = src.pair(0)
    fs = vqm.FrameSet([r], [d], src.bpc)   # host arrays
    with pytest.raises(vqm.VqmError) as e:
        vqm.Graph(0, None, vqm.VQM_METRIC_FLOAT_SSIM, fs, 8)
    assert e.value.rc == -errno.EINVAL
    assert "device memory" in vqm.vqm_last_error()
