"""Host-side checks of the C ABI library (no GPU needed).

The library loads without a GPU, exports every entry point ``include/vqm.h``
declares, and its host-only logic — the scale rule, the geometry and the gate,
argument errors — answers before any HIP call.
"""

import ctypes
import errno
import os
import re

import numpy as np
import pytest

import oracle
from full_reference_video_amd import vqm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vqm.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"VQM_API\s+[\w\s\*]*?\b(vqm_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for must in ("vqm_ssim_frame", "vqm_msssim_frame", "vqm_ctx_create", "vqm_ssim_submit",
                 "vqm_msssim_submit", "vqm_collect", "vqm_last_error", "vqm_debug_decimate"):
        assert must in names
    assert len(names) >= 17


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(vqm.LIB_PATH)
    missing = [n for n in declared_symbols() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_the_abi():
    for n in declared_symbols():
        if n in ("vqm_ctx_destroy", "vqm_graph_create", "vqm_graph_destroy"):
            continue  # Context() / Graph() and their close()
        assert hasattr(vqm, n) or hasattr(vqm.Context, n) or hasattr(vqm.Graph, n), n


def header_constants():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(VQM_\w+)\s+(-?\d+)\s*$", text, re.M)}


def test_abi_version():
    assert vqm.vqm_abi_version() == header_constants()["VQM_ABI_VERSION"] == 9


def test_graft_entry_check_matches_the_built_library():
    # build() ends with this check: the loaded library's ABI version against
    # the header's (a stale literal there once failed every build).
    import __graft_entry__
    assert __graft_entry__.header_abi_version() == header_constants()["VQM_ABI_VERSION"]
    __graft_entry__.check_loaded()


def test_binding_constants_match_the_header():
    consts = header_constants()
    for name in ("VQM_MAX_IN_FLIGHT", "VQM_MAX_BATCH", "VQM_MSSSIM_LCS", "VQM_SS2_MAX_IN_FLIGHT"):
        assert getattr(vqm, name) == consts[name], name
    # a float_ssim batch passes through three step launches before its
    # frames can be collected; the in-flight limit leaves room for more
    assert consts["VQM_MAX_IN_FLIGHT"] >= 4 * consts["VQM_MAX_BATCH"]


def test_scale_rule_matches_oracle():
    for w in list(range(1, 2000, 7)) + [3839, 3840, 7680, 32895, 32896]:
        for h in (1, 255, 383, 384, 481, 640, 1080, 2160, 4320, 32896):
            assert vqm.vqm_ssim_scale(w, h) == oracle.scale(w, h), (w, h)
    assert vqm.vqm_ssim_scale(0, 100) == 0


@pytest.mark.parametrize("w,h,s,dw,dh", [(576, 324, 1, 576, 324), (853, 481, 2, 427, 241),
                                         (1920, 1080, 4, 480, 270), (3840, 2160, 8, 480, 270)])
def test_geometry_of_the_workloads(w, h, s, dw, dh):
    assert vqm.vqm_ssim_geometry(w, h, 10) == (s, dw, dh)
    assert (oracle.decimated_dim(w, s), oracle.decimated_dim(h, s)) == (dw, dh)


def _rc(fn, *args):
    try:
        fn(*args)
    except vqm.VqmError as e:
        return e.rc
    return 0


def test_gate_agrees_with_oracle_without_a_gpu():
    # The gate answers -ENOTSUP before any HIP call, so this runs on the CPU.
    z = np.zeros(16, np.uint16)
    for (w, h) in [(10, 200), (200, 10), (11, 11), (12, 30), (2815, 2815), (2816, 2816),
                   (32896, 32896), (32895, 100), (3000, 43)]:
        s = oracle.scale(w, h)
        refused = s > 128 or oracle.decimated_dim(w, s) < 11 or oracle.decimated_dim(h, s) < 11
        got = vqm.lib().vqm_ssim_geometry(w, h, 10, None, None, None)
        assert got == (-errno.ENOTSUP if refused else 0), (w, h, got)
        if refused:  # the oracle's gate also answers before reading the planes
            assert oracle.ssim_rc(z, z, w, h, 10) == -errno.ENOTSUP


def test_argument_errors_before_any_hip_call():
    L = vqm.lib()
    a = np.zeros((20, 20), np.uint8)
    s = ctypes.c_double(123.0)
    p = a.ctypes.data
    assert L.vqm_ssim_frame(None, p, 20, 20, 8, ctypes.byref(s)) == -errno.EINVAL
    assert L.vqm_ssim_frame(p, p, 0, 20, 8, ctypes.byref(s)) == -errno.EINVAL
    assert L.vqm_ssim_frame(p, p, 20, 20, 7, ctypes.byref(s)) == -errno.EINVAL
    assert L.vqm_ssim_frame(p, p, 20, 20, 17, ctypes.byref(s)) == -errno.EINVAL
    assert L.vqm_ssim_frame(p, p, 65536, 65536, 8, ctypes.byref(s)) == -errno.EINVAL
    assert L.vqm_ssim_frame(p, p, 20, 20, 8, None) == -errno.EINVAL
    assert L.vqm_ssim_frame(p, p, 10, 20, 8, ctypes.byref(s)) == -errno.ENOTSUP
    assert L.vqm_msssim_frame(p, p, 175, 400, 8, ctypes.byref(s)) == -errno.ENOTSUP
    assert s.value == 123.0  # untouched on error
    assert "11x11" in vqm.vqm_last_error()
    assert L.vqm_ssim_frame_db(p, p, 20, 20, 8, ctypes.byref(s), None) == -errno.EINVAL
    assert L.vqm_collect(None, ctypes.byref(s), None) == -errno.EINVAL
    assert L.vqm_collect_db(None, ctypes.byref(s), None) == -errno.EINVAL
    assert L.vqm_ssim_submit(None, p, p, 20, 20, 8) == -errno.EINVAL
    arr = (ctypes.c_void_p * 2)(p, p)
    out = np.zeros(4, np.float32).ctypes.data
    assert L.vqm_debug_pyramid_batch(None, arr, arr, 2, 400, 400, 8, 2, out, out) == -errno.EINVAL


def test_graph_argument_errors_before_any_hip_call():
    L = vqm.lib()
    a = np.zeros((400, 400), np.uint8)
    p = a.ctypes.data
    arr = (ctypes.c_void_p * 2)(p, p)
    g = ctypes.c_void_p(7)
    out = ctypes.byref(g)
    F, M = vqm.VQM_METRIC_FLOAT_SSIM, vqm.VQM_METRIC_MS_SSIM
    assert L.vqm_graph_create(0, None, 2, arr, arr, 2, 400, 400, 8, 8, out) == -errno.EINVAL  # metric
    assert L.vqm_graph_create(0, None, F, None, arr, 2, 400, 400, 8, 8, out) == -errno.EINVAL
    assert L.vqm_graph_create(0, None, F, arr, arr, 0, 400, 400, 8, 8, out) == -errno.EINVAL
    big = (ctypes.c_void_p * (vqm.VQM_MAX_IN_FLIGHT + 1))(*([p] * (vqm.VQM_MAX_IN_FLIGHT + 1)))
    assert L.vqm_graph_create(0, None, F, big, big, vqm.VQM_MAX_IN_FLIGHT + 1, 400, 400, 8, 8,
                              out) == -errno.EINVAL
    assert L.vqm_graph_create(0, None, F, arr, arr, 2, 400, 400, 8, 0, out) == -errno.EINVAL
    assert L.vqm_graph_create(0, None, F, arr, arr, 2, 400, 400, 8, vqm.VQM_MAX_BATCH + 1, out) == -errno.EINVAL
    assert L.vqm_graph_create(0, None, F, arr, arr, 2, 400, 400, 7, 8, out) == -errno.EINVAL
    assert L.vqm_graph_create(0, None, F, arr, arr, 2, 10, 400, 8, 8, out) == -errno.ENOTSUP  # the gate
    assert L.vqm_graph_create(0, None, M, arr, arr, 2, 175, 400, 8, 8, out) == -errno.ENOTSUP
    assert g.value is None  # *out is cleared on error
    assert L.vqm_graph_create(0, None, F, arr, arr, 2, 400, 400, 8, 8, None) == -errno.EINVAL
    assert L.vqm_graph_launch(None) == -errno.EINVAL
    s = ctypes.c_double()
    assert L.vqm_graph_collect(None, ctypes.byref(s), None, None) == -errno.EINVAL
    L.vqm_graph_destroy(None)  # a no-op


def test_binding_checks_sample_size_and_shape():
    a8 = np.zeros((20, 20), np.uint8)
    a16 = np.zeros((20, 20), np.uint16)
    with pytest.raises(TypeError):
        vqm.vqm_ssim_frame(a8, a8, 10)
    with pytest.raises(TypeError):
        vqm.vqm_ssim_frame(a16, a16, 8)
    with pytest.raises(ValueError):
        vqm.vqm_ssim_frame(a8, np.zeros((20, 21), np.uint8), 8)
    with pytest.raises(ValueError):
        vqm.vqm_ssim_frame(a8[:, ::2], a8[:, ::2], 8)


@pytest.mark.skipif(os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK),
                    reason="a GPU is present")
def test_no_device_is_enodev():
    a = np.zeros((400, 400), np.uint8)
    assert _rc(vqm.vqm_ssim_frame, a, a, 8) == -errno.ENODEV
    assert _rc(vqm.Context, 0, None) == -errno.ENODEV


def test_plane_dims_match_oracle():
    for (w, h) in [(1920, 1080), (853, 481), (576, 324), (1, 1), (7, 9)]:
        for chroma in (vqm.VQM_CHROMA_420, vqm.VQM_CHROMA_422, vqm.VQM_CHROMA_444):
            for plane in range(3):
                assert vqm.vqm_plane_dims(w, h, chroma, plane) == oracle.plane_dims(w, h, chroma, plane)
    L = vqm.lib()
    a, b = ctypes.c_int(), ctypes.c_int()
    assert L.vqm_plane_dims(10, 10, 3, 1, ctypes.byref(a), ctypes.byref(b)) == -errno.EINVAL
    assert L.vqm_plane_dims(10, 10, 0, 3, ctypes.byref(a), ctypes.byref(b)) == -errno.EINVAL


def test_yuv_gate_refuses_before_any_hip_call():
    # 576x324 4:2:0: the 288x162 chroma planes are below MS-SSIM's
    # 11 x 16 rows, so the whole call is refused, naming the plane.
    w, h = 576, 324
    planes = [np.zeros(oracle.plane_dims(w, h, 0, p)[::-1], np.uint8) for p in range(3)]
    with pytest.raises(vqm.VqmError) as e:
        vqm.vqm_msssim_frame_yuv(planes, planes, 8, vqm.VQM_CHROMA_420)
    assert e.value.rc == -errno.ENOTSUP
    assert "plane 1" in vqm.vqm_last_error()
    with pytest.raises(ValueError):  # wrong chroma size for the layout
        vqm.vqm_ssim_frame_yuv(planes, planes, 8, vqm.VQM_CHROMA_444)


def test_noalloc_refuses_oversized_and_bad_frames_before_any_hip_call():
    # The allocation-free entry point checks its arguments, the gate and its
    # fixed scratch size on the host first; none of these touches the GPU.
    lib = ctypes.CDLL(vqm.LIB_PATH)
    f = lib.vqm_ssim_frame_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p]
    dummy = ctypes.c_void_p(0x1000)
    # 65535 x 400 decimates by 2 to 32768 x 200: two fp32 planes of 25 MiB
    assert f(dummy, dummy, 65535, 400, 8, dummy, None) == -errno.ENOSPC
    assert "scratch" in vqm.vqm_last_error()
    assert f(dummy, dummy, 3840, 2160, 10, None, None) == -errno.EINVAL      # no score buffer
    assert f(None, dummy, 3840, 2160, 10, dummy, None) == -errno.EINVAL      # no plane
    assert f(dummy, dummy, 3840, 2160, 7, dummy, None) == -errno.EINVAL      # depth
    assert f(dummy, dummy, 100, 8, 8, dummy, None) == -errno.ENOTSUP        # below the window
    # 8K (scale 17) needs about 1 MiB of the 8 MiB array: past the size check
    # (here it then fails at the device or pointer checks instead)
    assert header_constants()["VQM_NOALLOC_SCRATCH_BYTES"] == 8 << 20
    assert f(dummy, dummy, 7680, 4320, 10, dummy, None) not in (0, -errno.ENOSPC)


def test_ss2_chain_refuses_bad_arguments_before_any_hip_call():
    # Every check of the chain's entry points precedes the first HIP call.
    L = vqm.lib()
    dummy = ctypes.c_void_p(0x1000)
    coef = np.array([0.5, 0.25, -0.125, 0.0625], np.float32)
    bad = np.array([0.5, np.inf, 0.0, 0.0], np.float32)
    sums = np.zeros(6 * 3 * 6, np.float64)
    sp = sums.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    arr = (ctypes.c_void_p * 3)(dummy, dummy, dummy)
    f = L.vqm_ss2_scale_sums
    assert f(None, arr, 1, 64, 64, 2, coef.ctypes.data, sp) == -errno.EINVAL
    assert f(arr, arr, 0, 64, 64, 2, coef.ctypes.data, sp) == -errno.EINVAL       # channels
    assert f(arr, arr, 4, 64, 64, 2, coef.ctypes.data, sp) == -errno.EINVAL
    assert f(arr, arr, 1, 64, 64, 0, coef.ctypes.data, sp) == -errno.EINVAL       # scales
    assert f(arr, arr, 1, 64, 64, 7, coef.ctypes.data, sp) == -errno.EINVAL
    assert f(arr, arr, 1, 0, 64, 2, coef.ctypes.data, sp) == -errno.EINVAL        # size
    assert f(arr, arr, 1, 65536, 65536, 2, coef.ctypes.data, sp) == -errno.EINVAL
    assert f(arr, arr, 1, 64, 64, 2, bad.ctypes.data, sp) == -errno.EINVAL        # coefficients
    assert "coefficient 1" in vqm.vqm_last_error()
    assert f(arr, arr, 1, 64, 64, 2, None, sp) == -errno.EINVAL
    assert f(arr, arr, 1, 64, 64, 2, coef.ctypes.data, None) == -errno.EINVAL
    assert L.vqm_ss2_blur(None, dummy, 8, 8, coef.ctypes.data) == -errno.EINVAL
    assert L.vqm_ss2_blur(dummy, dummy, 8, -1, coef.ctypes.data) == -errno.EINVAL
    assert L.vqm_ss2_blur(dummy, dummy, 8, 8, bad.ctypes.data) == -errno.EINVAL
    assert L.vqm_ss2_downsample(dummy, None, 8, 8) == -errno.EINVAL
    assert L.vqm_ss2_downsample(dummy, dummy, 0, 8) == -errno.EINVAL
    assert L.vqm_debug_ss2_blurred(arr, arr, 1, 64, 64, 1, coef.ctypes.data, None, sp) == -errno.EINVAL
    assert L.vqm_debug_ss2_blurred(arr, arr, 1, 64, 64, 1, coef.ctypes.data, (ctypes.c_void_p * 1)(None),
                                   sp) == -errno.EINVAL
    assert L.vqm_debug_ss2_blurred(arr, arr, 1, 64, 64, 7, coef.ctypes.data, arr, sp) == -errno.EINVAL
    # submit and collect on a context: the same checks, and NULL context
    ctx = ctypes.c_void_p(0x2000)  # never dereferenced: every check below fails first
    g = L.vqm_ss2_submit
    assert g(None, arr, arr, 1, 64, 64, 2, coef.ctypes.data) == -errno.EINVAL
    assert g(ctx, None, arr, 1, 64, 64, 2, coef.ctypes.data) == -errno.EINVAL
    assert g(ctx, arr, arr, 4, 64, 64, 2, coef.ctypes.data) == -errno.EINVAL
    assert g(ctx, arr, arr, 1, 64, 64, 7, coef.ctypes.data) == -errno.EINVAL
    assert g(ctx, arr, arr, 1, 64, 0, 2, coef.ctypes.data) == -errno.EINVAL
    assert g(ctx, arr, arr, 1, 64, 64, 2, bad.ctypes.data) == -errno.EINVAL
    assert g(ctx, (ctypes.c_void_p * 1)(None), arr, 1, 64, 64, 2, coef.ctypes.data) == -errno.EINVAL
    assert L.vqm_ss2_collect(None, sp) == -errno.EINVAL
    assert L.vqm_ss2_collect(ctx, None) == -errno.EINVAL
    assert L.vqm_ss2_in_flight(None) == 0
    t = ctypes.c_double()
    assert L.vqm_debug_valu_probe(0, 100, 1, ctypes.byref(t)) == -errno.EINVAL   # waves per SIMD
    assert L.vqm_debug_valu_probe(33, 100, 1, ctypes.byref(t)) == -errno.EINVAL
    assert L.vqm_debug_valu_probe(4, 0, 1, ctypes.byref(t)) == -errno.EINVAL     # iterations
    assert L.vqm_debug_valu_probe(4, 100, 0, ctypes.byref(t)) == -errno.EINVAL   # repetitions
    assert L.vqm_debug_valu_probe(4, 100, 1, None) == -errno.EINVAL
    c = np.zeros(4, np.float32)
    assert L.vqm_ss2_cascade_coefficients(0.0, c.ctypes.data) == -errno.EINVAL
    assert L.vqm_ss2_cascade_coefficients(1.5, None) == -errno.EINVAL
