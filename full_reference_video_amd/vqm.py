"""Thin ctypes binding of ``libvqm.so`` (the C ABI of ``include/vqm.h``).

Argument marshalling only: every step of the scoring runs in the HIP library.
The names match the C entry points.  Planes may be numpy arrays (host memory)
or torch tensors (host, pinned host or device memory): uint8 samples when
``bpc == 8``, 16-bit samples otherwise (numpy uint16; torch int16/uint16
tensors are passed by their bytes).  Shapes are ``(h, w)``, C-contiguous.

If the library has not been built this module raises on first use; there is
no fallback path.
"""

from __future__ import annotations

import collections
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvqm.so")

VQM_MAX_IN_FLIGHT = 192
VQM_MAX_BATCH = 32
VQM_MSSSIM_LCS = 15
VQM_SS2_MAX_IN_FLIGHT = 4
VQM_METRIC_FLOAT_SSIM = 0
VQM_METRIC_MS_SSIM = 1
VQM_KERNEL_SSIM_STEP = 0
VQM_KERNEL_SSIM_DRAIN = 1
VQM_KERNEL_MSSSIM_LEVEL1 = 2
VQM_KERNEL_MSSSIM_COARSE = 3
VQM_CHROMA_420 = 0
VQM_CHROMA_422 = 1
VQM_CHROMA_444 = 2


class VqmError(RuntimeError):
    """A negative errno returned by the library, with its message."""

    def __init__(self, rc: int, where: str, msg: str):
        name = os.strerror(-rc) if rc < 0 else str(rc)
        super().__init__(f"{where}: {rc} ({name}): {msg}")
        self.rc = rc


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "or python -m full_reference_video_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_void_p, c_double_p = ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        c_int_p = ctypes.POINTER(ctypes.c_int)
        L.vqm_abi_version.restype = c_int
        L.vqm_ssim_scale.argtypes = [c_int, c_int]
        L.vqm_ssim_geometry.argtypes = [c_int, c_int, c_int, c_int_p, c_int_p, c_int_p]
        for n in ("vqm_ssim_frame", "vqm_msssim_frame"):
            getattr(L, n).argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_double_p]
        L.vqm_msssim_frame_lcs.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_double_p, c_double_p]
        L.vqm_ssim_frame_db.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_double_p, c_double_p]
        L.vqm_plane_dims.argtypes = [c_int, c_int, c_int, c_int, c_int_p, c_int_p]
        for n in ("vqm_ssim_frame_yuv", "vqm_msssim_frame_yuv"):
            getattr(L, n).argtypes = [ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p), c_int, c_int, c_int, c_int,
                                      c_double_p, c_double_p]
        L.vqm_ctx_create.argtypes = [c_int, c_void_p, ctypes.POINTER(c_void_p)]
        L.vqm_ctx_destroy.argtypes = [c_void_p]
        L.vqm_ctx_destroy.restype = None
        for n in ("vqm_ssim_submit", "vqm_msssim_submit"):
            getattr(L, n).argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int]
        for n in ("vqm_ssim_submit_batch", "vqm_msssim_submit_batch"):
            getattr(L, n).argtypes = [c_void_p, ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p), c_int,
                                      c_int, c_int, c_int]
        L.vqm_collect.argtypes = [c_void_p, c_double_p, c_double_p]
        L.vqm_collect_db.argtypes = [c_void_p, c_double_p, c_double_p]
        L.vqm_score_frames.argtypes = [ctypes.POINTER(c_void_p), c_int, c_int, ctypes.POINTER(c_void_p),
                                       ctypes.POINTER(c_void_p), c_int, c_int, c_int, c_int, c_int, c_int,
                                       c_double_p, c_double_p, c_double_p]
        L.vqm_in_flight.argtypes = [c_void_p]
        L.vqm_ctx_set_timing.argtypes = [c_void_p, c_int]
        L.vqm_ctx_kernel_time.argtypes = [c_void_p, c_int, c_double_p, c_int_p, c_int_p]
        L.vqm_debug_decimate.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                         c_void_p, c_void_p]
        L.vqm_debug_pyramid.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                        c_void_p, c_void_p]
        L.vqm_debug_pyramid_batch.argtypes = [c_void_p, ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p), c_int,
                                              c_int, c_int, c_int, c_int, c_void_p, c_void_p]
        L.vqm_graph_create.argtypes = [c_int, c_void_p, c_int, ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p),
                                       c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(c_void_p)]
        L.vqm_graph_launch.argtypes = [c_void_p]
        L.vqm_graph_collect.argtypes = [c_void_p, c_double_p, c_double_p, c_double_p]
        L.vqm_graph_destroy.argtypes = [c_void_p]
        L.vqm_graph_destroy.restype = None
        L.vqm_ssim_frame_noalloc.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p]
        L.vqm_ss2_channel_sums.argtypes = [ctypes.POINTER(c_void_p), c_int, c_int, c_int, c_double_p]
        L.vqm_debug_pair_ops.argtypes = [c_int, c_void_p, c_void_p, c_void_p, c_int]
        L.vqm_ss2_blur.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p]
        L.vqm_ss2_downsample.argtypes = [c_void_p, c_void_p, c_int, c_int]
        L.vqm_ss2_scale_sums.argtypes = [ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p), c_int, c_int, c_int,
                                         c_int, c_void_p, c_double_p]
        L.vqm_ss2_cascade_coefficients.argtypes = [ctypes.c_double, c_void_p]
        L.vqm_ss2_submit.argtypes = [c_void_p, ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p), c_int, c_int,
                                     c_int, c_int, c_void_p]
        L.vqm_ss2_collect.argtypes = [c_void_p, c_double_p]
        L.vqm_ss2_in_flight.argtypes = [c_void_p]
        L.vqm_debug_ss2_blurred.argtypes = [ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p), c_int, c_int, c_int,
                                            c_int, c_void_p, ctypes.POINTER(c_void_p), c_double_p]
        L.vqm_debug_read_probe.argtypes = [c_void_p, ctypes.c_longlong, c_int, c_double_p]
        L.vqm_debug_valu_probe.argtypes = [c_int, c_int, c_int, c_double_p]
        L.vqm_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def vqm_last_error() -> str:
    return lib().vqm_last_error().decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise VqmError(rc, where, vqm_last_error())


def _plane(a, bpc: int):
    """(pointer, w, h, keepalive) of a plane; checks shape, layout and sample size."""
    want = 1 if bpc == 8 else 2
    if isinstance(a, np.ndarray):
        if a.ndim != 2 or not a.flags.c_contiguous:
            raise ValueError("plane must be a C-contiguous 2-D array")
        if a.itemsize != want:
            raise TypeError(f"bpc {bpc} needs {want}-byte samples, got {a.dtype}")
        return a.ctypes.data, a.shape[1], a.shape[0], a
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(a, torch.Tensor):
        if a.dim() != 2 or not a.is_contiguous():
            raise ValueError("plane must be a contiguous 2-D tensor")
        if a.element_size() != want:
            raise TypeError(f"bpc {bpc} needs {want}-byte samples, got {a.dtype}")
        return a.data_ptr(), a.shape[1], a.shape[0], a
    raise TypeError(f"unsupported plane type {type(a)!r}")


def _pair(ref, dis, bpc):
    pr, w, h, kr = _plane(ref, bpc)
    pd, w2, h2, kd = _plane(dis, bpc)
    if (w, h) != (w2, h2):
        raise ValueError(f"ref is {w}x{h} but dis is {w2}x{h2}")
    return pr, pd, w, h, (kr, kd)


def vqm_abi_version() -> int:
    return lib().vqm_abi_version()


def vqm_ssim_scale(w: int, h: int) -> int:
    return lib().vqm_ssim_scale(int(w), int(h))


def vqm_ssim_geometry(w: int, h: int, bpc: int):
    s, dw, dh = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().vqm_ssim_geometry(int(w), int(h), int(bpc), ctypes.byref(s), ctypes.byref(dw),
                                   ctypes.byref(dh)), "vqm_ssim_geometry")
    return s.value, dw.value, dh.value


def vqm_ssim_frame(ref, dis, bpc: int) -> float:
    pr, pd, w, h, _ = _pair(ref, dis, bpc)
    score = ctypes.c_double()
    _check(lib().vqm_ssim_frame(pr, pd, w, h, int(bpc), ctypes.byref(score)), "vqm_ssim_frame")
    return score.value


def vqm_ssim_frame_db(ref, dis, bpc: int):
    """(score, decibel form) of one frame pair."""
    pr, pd, w, h, _ = _pair(ref, dis, bpc)
    score, db = ctypes.c_double(), ctypes.c_double()
    _check(lib().vqm_ssim_frame_db(pr, pd, w, h, int(bpc), ctypes.byref(score), ctypes.byref(db)),
           "vqm_ssim_frame_db")
    return score.value, db.value


def vqm_plane_dims(w: int, h: int, chroma: int, plane: int):
    """(width, height) of plane 0..2 of a w x h picture in a chroma layout."""
    pw, ph = ctypes.c_int(), ctypes.c_int()
    _check(lib().vqm_plane_dims(int(w), int(h), int(chroma), int(plane), ctypes.byref(pw), ctypes.byref(ph)),
           "vqm_plane_dims")
    return pw.value, ph.value


def _yuv(refs, diss, bpc: int, chroma: int):
    if len(refs) != 3 or len(diss) != 3:
        raise ValueError("three planes (Y, Cb, Cr) per picture")
    pr = (ctypes.c_void_p * 3)()
    pd = (ctypes.c_void_p * 3)()
    keep = []
    w = h = None
    for p in range(3):
        a, b, pw, ph, k = _pair(refs[p], diss[p], bpc)
        if p == 0:
            w, h = pw, ph
        elif (pw, ph) != vqm_plane_dims(w, h, chroma, p):
            raise ValueError(f"plane {p} is {pw}x{ph}, the layout needs {vqm_plane_dims(w, h, chroma, p)}")
        pr[p], pd[p] = a, b
        keep.append(k)
    return pr, pd, w, h, keep


def vqm_ssim_frame_yuv(refs, diss, bpc: int, chroma: int):
    """(scores[3], decibel forms[3]) of the Y, Cb and Cr planes of a frame pair."""
    pr, pd, w, h, _keep = _yuv(refs, diss, bpc, chroma)
    scores, db = np.empty(3, np.float64), np.empty(3, np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(lib().vqm_ssim_frame_yuv(pr, pd, w, h, int(bpc), int(chroma), scores.ctypes.data_as(dp),
                                    db.ctypes.data_as(dp)), "vqm_ssim_frame_yuv")
    return scores, db


def vqm_msssim_frame_yuv(refs, diss, bpc: int, chroma: int):
    """(scores[3], per-level means [3, 15]) of the Y, Cb and Cr planes."""
    pr, pd, w, h, _keep = _yuv(refs, diss, bpc, chroma)
    scores, lcs = np.empty(3, np.float64), np.empty((3, VQM_MSSSIM_LCS), np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(lib().vqm_msssim_frame_yuv(pr, pd, w, h, int(bpc), int(chroma), scores.ctypes.data_as(dp),
                                      lcs.ctypes.data_as(dp)), "vqm_msssim_frame_yuv")
    return scores, lcs


def vqm_msssim_frame(ref, dis, bpc: int) -> float:
    pr, pd, w, h, _ = _pair(ref, dis, bpc)
    score = ctypes.c_double()
    _check(lib().vqm_msssim_frame(pr, pd, w, h, int(bpc), ctypes.byref(score)), "vqm_msssim_frame")
    return score.value


def vqm_msssim_frame_lcs(ref, dis, bpc: int):
    pr, pd, w, h, _ = _pair(ref, dis, bpc)
    score = ctypes.c_double()
    lcs = np.empty(VQM_MSSSIM_LCS, np.float64)
    _check(lib().vqm_msssim_frame_lcs(pr, pd, w, h, int(bpc), ctypes.byref(score),
                                      lcs.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
           "vqm_msssim_frame_lcs")
    return score.value, lcs


def vqm_ssim_frame_noalloc(ref, dis, bpc: int, score, stream=None) -> None:
    """Enqueue float_ssim of one device-resident frame pair with no allocation.

    ``score`` is a float64 tensor of at least one element in device memory (or
    pinned host memory) that receives the score once ``stream`` (a
    ``torch.cuda.Stream``, a raw handle, or None for the legacy default
    stream) reaches this point; the call does not wait.
    """
    pr, pd, w, h, _ = _pair(ref, dis, bpc)
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(score, torch.Tensor):
        if score.dtype != torch.float64 or score.numel() < 1:
            raise TypeError("score must be a float64 tensor with at least one element")
        sp = score.data_ptr()
    elif isinstance(score, int):
        sp = score
    else:
        raise TypeError(f"unsupported score buffer {type(score)!r}")
    _check(lib().vqm_ssim_frame_noalloc(pr, pd, w, h, int(bpc), sp, _stream_handle(stream)),
           "vqm_ssim_frame_noalloc")


SS2_PLANES = ("img1", "img2", "mu1", "mu2", "s11", "s22", "s12")


def vqm_ss2_channel_sums(channels) -> np.ndarray:
    """The six ssimulacra2 sums per channel (array [nch, 6]).

    ``channels`` is a list of 1..3 channels, each a sequence of seven float32
    device tensors in the order of ``SS2_PLANES``, all of one (h, w) shape.
    """
    import torch
    nch = len(channels)
    ptrs = (ctypes.c_void_p * (7 * nch))()
    h = w = None
    for c, planes in enumerate(channels):
        if len(planes) != 7:
            raise ValueError("seven planes per channel")
        for p, t in enumerate(planes):
            if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous():
                raise TypeError("planes are contiguous 2-D float32 tensors")
            if h is None:
                h, w = t.shape
            elif tuple(t.shape) != (h, w):
                raise ValueError("all planes must have one shape")
            ptrs[c * 7 + p] = t.data_ptr()
    out = np.empty((nch, 6), np.float64)
    _check(lib().vqm_ss2_channel_sums(ptrs, nch, int(w), int(h), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
           "vqm_ss2_channel_sums")
    return out


def _f32_plane(t, what):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous():
        raise TypeError(f"{what}: a contiguous 2-D float32 device tensor")
    return t


def _coef_array(coef) -> np.ndarray:
    c = np.ascontiguousarray(coef, np.float32)
    if c.shape != (4,):
        raise ValueError("four recursion coefficients (B, a1, a2, a3)")
    return c


def vqm_ss2_cascade_coefficients(sigma: float) -> np.ndarray:
    """(B, a1, a2, a3) of the library's recursive bell of variance sigma^2."""
    out = np.empty(4, np.float32)
    _check(lib().vqm_ss2_cascade_coefficients(float(sigma), out.ctypes.data), "vqm_ss2_cascade_coefficients")
    return out


def vqm_ss2_blur(plane, coef, out=None):
    """The recursive blur (rows, then columns) of a float32 device plane;
    ``out`` (default: a new tensor) may be ``plane`` itself."""
    import torch
    plane = _f32_plane(plane, "plane")
    out = torch.empty_like(plane) if out is None else _f32_plane(out, "out")
    if out.shape != plane.shape:
        raise ValueError("out must have the plane's shape")
    c = _coef_array(coef)
    h, w = plane.shape
    _check(lib().vqm_ss2_blur(plane.data_ptr(), out.data_ptr(), int(w), int(h), c.ctypes.data), "vqm_ss2_blur")
    return out


def vqm_ss2_downsample(plane):
    """The chain's 2x2 downsample of a float32 device plane (sizes round up)."""
    import torch
    plane = _f32_plane(plane, "plane")
    h, w = plane.shape
    out = torch.empty(((h + 1) // 2, (w + 1) // 2), dtype=torch.float32, device=plane.device)
    _check(lib().vqm_ss2_downsample(plane.data_ptr(), out.data_ptr(), int(w), int(h)), "vqm_ss2_downsample")
    return out


def _ss2_planes(ref_planes, dis_planes):
    """(ref pointer array, dis pointer array, nch, w, h) of a chain frame."""
    nch = len(ref_planes)
    if nch != len(dis_planes):
        raise ValueError("one reference and one distorted plane per channel")
    rp, dp = (ctypes.c_void_p * max(nch, 1))(), (ctypes.c_void_p * max(nch, 1))()
    h = w = None
    for c in range(nch):
        for arr, t, what in ((rp, ref_planes[c], "reference"), (dp, dis_planes[c], "distorted")):
            _f32_plane(t, what)
            if h is None:
                h, w = t.shape
            elif tuple(t.shape) != (h, w):
                raise ValueError("all planes must have one shape")
            arr[c] = t.data_ptr()
    return rp, dp, nch, int(w or 0), int(h or 0)


def vqm_ss2_scale_sums(ref_planes, dis_planes, nscales: int, coef) -> np.ndarray:
    """The six sums per channel at every scale of the per-scale chain,
    array [nscales, nch, 6]; ``ref_planes``/``dis_planes`` hold 1..3 float32
    device tensors of one (h, w) shape."""
    rp, dp, nch, w, h = _ss2_planes(ref_planes, dis_planes)
    cf = _coef_array(coef)
    out = np.empty((max(int(nscales), 1), max(nch, 1), 6), np.float64)
    _check(lib().vqm_ss2_scale_sums(rp, dp, nch, w, h, int(nscales), cf.ctypes.data,
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))), "vqm_ss2_scale_sums")
    return out


def vqm_debug_ss2_blurred(ref_planes, dis_planes, coef, nscales: int = 1):
    """The chain with its blurred planes: (sums [nscales, nch, 6], blurred)
    where blurred[s] is a device tensor [nch, 5, h_s, w_s] holding mu1, mu2,
    s11, s22, s12 of each channel at scale s."""
    import torch
    nch = len(ref_planes)
    if nch != len(dis_planes) or nch < 1:
        raise ValueError("one reference and one distorted plane per channel")
    for t in list(ref_planes) + list(dis_planes):
        _f32_plane(t, "plane")
        if t.shape != ref_planes[0].shape:
            raise ValueError("all planes must have one shape")
    h, w = ref_planes[0].shape
    ns = int(nscales)
    dims = [(h, w)]
    for _ in range(1, max(ns, 1)):
        dims.append(((dims[-1][0] + 1) // 2, (dims[-1][1] + 1) // 2))
    per_ch = sum(5 * a * b for a, b in dims)
    flat = torch.empty((nch, per_ch), dtype=torch.float32, device=ref_planes[0].device)
    arr = ctypes.c_void_p * nch
    rp, dp = arr(*[t.data_ptr() for t in ref_planes]), arr(*[t.data_ptr() for t in dis_planes])
    op = arr(*[flat[c].data_ptr() for c in range(nch)])
    cf = _coef_array(coef)
    sums = np.empty((max(ns, 1), nch, 6), np.float64)
    _check(lib().vqm_debug_ss2_blurred(rp, dp, nch, int(w), int(h), ns, cf.ctypes.data, op,
                                       sums.ctypes.data_as(ctypes.POINTER(ctypes.c_double))), "vqm_debug_ss2_blurred")
    planes, off = [], 0
    for a, b in dims:
        planes.append(flat[:, off:off + 5 * a * b].view(nch, 5, a, b))
        off += 5 * a * b
    return sums, planes


def vqm_debug_pair_ops(op: int, a, b) -> np.ndarray:
    """op (0 two_sum, 1 two_prod, 2 ff_add, 3 ff_mul, 4 ff_div) on the device
    over float32 pair arrays a, b of shape [n, 2] (hi, lo); returns [n, 2]."""
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    if a.ndim != 2 or a.shape[1] != 2 or a.shape != b.shape:
        raise ValueError("pair arrays of shape [n, 2]")
    out = np.empty_like(a)
    _check(lib().vqm_debug_pair_ops(int(op), a.ctypes.data, b.ctypes.data, out.ctypes.data, a.shape[0]),
           "vqm_debug_pair_ops")
    return out


def vqm_debug_valu_probe(waves_per_simd: int = 8, iters: int = 20000, reps: int = 5) -> float:
    """TFLOP/s of plain (non-packed) fp32 FMA chains on the vector units."""
    t = ctypes.c_double()
    _check(lib().vqm_debug_valu_probe(int(waves_per_simd), int(iters), int(reps), ctypes.byref(t)),
           "vqm_debug_valu_probe")
    return t.value


def vqm_debug_read_probe(buf, reps: int = 20) -> float:
    """Mean milliseconds of the library's streaming read over a device
    tensor's bytes."""
    ms = ctypes.c_double()
    _check(lib().vqm_debug_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), int(reps),
                                      ctypes.byref(ms)), "vqm_debug_read_probe")
    return ms.value


def _stream_handle(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    handle = getattr(stream, "cuda_stream", None)  # torch.cuda.Stream on ROCm
    if handle is None:
        raise TypeError(f"unsupported stream {stream!r}")
    return int(handle)


class Context:
    """A ``vqm_ctx``: one device, one stream, up to VQM_MAX_IN_FLIGHT frames in flight."""

    def __init__(self, device: int = 0, stream=None):
        self._h = ctypes.c_void_p()
        _check(lib().vqm_ctx_create(int(device), _stream_handle(stream), ctypes.byref(self._h)),
               "vqm_ctx_create")
        # Inputs of frames in flight stay referenced until collected (pinned
        # or device planes are read after submit returns).
        self._inflight = collections.deque()
        # ssimulacra2 chain frames in flight: (planes, nscales, nch)
        self._ss2_inflight = collections.deque()

    def close(self):
        if self._h:
            lib().vqm_ctx_destroy(self._h)
            self._h = ctypes.c_void_p()
            self._inflight.clear()
            self._ss2_inflight.clear()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def vqm_ssim_submit(self, ref, dis, bpc: int):
        pr, pd, w, h, keep = _pair(ref, dis, bpc)
        _check(lib().vqm_ssim_submit(self._h, pr, pd, w, h, int(bpc)), "vqm_ssim_submit")
        self._inflight.append(keep)

    def vqm_msssim_submit(self, ref, dis, bpc: int):
        pr, pd, w, h, keep = _pair(ref, dis, bpc)
        _check(lib().vqm_msssim_submit(self._h, pr, pd, w, h, int(bpc)), "vqm_msssim_submit")
        self._inflight.append(keep)

    def _batch(self, fn, name, refs, diss, bpc):
        if len(refs) != len(diss):
            raise ValueError("refs and dis differ in length")
        n = len(refs)
        if not 1 <= n <= VQM_MAX_BATCH:
            raise ValueError(f"batch of {n} frames outside 1..{VQM_MAX_BATCH}")
        pr = (ctypes.c_void_p * n)()
        pd = (ctypes.c_void_p * n)()
        keep = []
        w = h = None
        for i, (r, d) in enumerate(zip(refs, diss)):
            a, b, fw, fh, k = _pair(r, d, bpc)
            if w is None:
                w, h = fw, fh
            elif (fw, fh) != (w, h):
                raise ValueError("frames of one batch must share their size")
            pr[i], pd[i] = a, b
            keep.append(k)
        _check(fn(self._h, pr, pd, n, w, h, int(bpc)), name)
        self._inflight.extend(keep)

    def vqm_ssim_submit_batch(self, refs, diss, bpc: int):
        self._batch(lib().vqm_ssim_submit_batch, "vqm_ssim_submit_batch", refs, diss, bpc)

    def vqm_msssim_submit_batch(self, refs, diss, bpc: int):
        self._batch(lib().vqm_msssim_submit_batch, "vqm_msssim_submit_batch", refs, diss, bpc)

    def vqm_collect(self, want_lcs: bool = False):
        score = ctypes.c_double()
        lcs = np.full(VQM_MSSSIM_LCS, np.nan)
        _check(lib().vqm_collect(self._h, ctypes.byref(score),
                                 lcs.ctypes.data_as(ctypes.POINTER(ctypes.c_double))), "vqm_collect")
        if self._inflight:
            self._inflight.popleft()
        return (score.value, lcs) if want_lcs else score.value

    def vqm_collect_db(self):
        """(score, decibel form) of the oldest frame in flight."""
        score, db = ctypes.c_double(), ctypes.c_double()
        _check(lib().vqm_collect_db(self._h, ctypes.byref(score), ctypes.byref(db)), "vqm_collect_db")
        if self._inflight:
            self._inflight.popleft()
        return score.value, db.value

    def vqm_in_flight(self) -> int:
        return lib().vqm_in_flight(self._h)

    def vqm_ss2_submit(self, ref_planes, dis_planes, nscales: int, coef):
        """Enqueue one frame of the per-scale chain (planes as
        vqm_ss2_scale_sums's) on its own slot stream, without waiting."""
        rp, dp, nch, w, h = _ss2_planes(ref_planes, dis_planes)
        cf = _coef_array(coef)
        _check(lib().vqm_ss2_submit(self._h, rp, dp, nch, w, h, int(nscales), cf.ctypes.data), "vqm_ss2_submit")
        self._ss2_inflight.append((list(ref_planes) + list(dis_planes), int(nscales), nch))

    def vqm_ss2_collect(self) -> np.ndarray:
        """The oldest chain frame's sums, array [nscales, nch, 6]."""
        ns, nch = self._ss2_inflight[0][1:] if self._ss2_inflight else (1, 1)
        out = np.full((ns, nch, 6), np.nan)
        _check(lib().vqm_ss2_collect(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
               "vqm_ss2_collect")
        self._ss2_inflight.popleft()
        return out

    def vqm_ss2_in_flight(self) -> int:
        return lib().vqm_ss2_in_flight(self._h)

    def vqm_ctx_set_timing(self, enable: bool):
        _check(lib().vqm_ctx_set_timing(self._h, 1 if enable else 0), "vqm_ctx_set_timing")

    def vqm_ctx_kernel_time(self, kernel_class: int):
        """(total_ms, launches, frames) of one kernel class since timing was switched on."""
        ms, n, f = ctypes.c_double(), ctypes.c_int(), ctypes.c_int()
        _check(lib().vqm_ctx_kernel_time(self._h, int(kernel_class), ctypes.byref(ms), ctypes.byref(n),
                                         ctypes.byref(f)), "vqm_ctx_kernel_time")
        return ms.value, n.value, f.value

    def vqm_debug_decimate(self, ref, dis, bpc: int, scale: int = 0):
        pr, pd, w, h, _ = _pair(ref, dis, bpc)
        if scale == 0:
            _, dw, dh = vqm_ssim_geometry(w, h, bpc)
        else:
            dw, dh = -(-w // scale), -(-h // scale)
        out_r = np.empty((dh, dw), np.float32)
        out_d = np.empty((dh, dw), np.float32)
        _check(lib().vqm_debug_decimate(self._h, pr, pd, w, h, int(bpc), int(scale), out_r.ctypes.data,
                                        out_d.ctypes.data), "vqm_debug_decimate")
        return out_r, out_d

    def vqm_debug_pyramid(self, ref, dis, bpc: int, level: int):
        pr, pd, w, h, _ = _pair(ref, dis, bpc)
        lw, lh = w >> (level - 1), h >> (level - 1)
        out_r = np.empty((lh, lw), np.float32)
        out_d = np.empty((lh, lw), np.float32)
        _check(lib().vqm_debug_pyramid(self._h, pr, pd, w, h, int(bpc), int(level), out_r.ctypes.data,
                                       out_d.ctypes.data), "vqm_debug_pyramid")
        return out_r, out_d


    def vqm_debug_pyramid_batch(self, refs, diss, bpc: int, level: int):
        """Level `level` of each frame's pyramid, built as one batch: two
        arrays of shape (n, lh, lw)."""
        if len(refs) != len(diss):
            raise ValueError("refs and dis differ in length")
        n = len(refs)
        if not 1 <= n <= VQM_MAX_BATCH:
            raise ValueError(f"batch of {n} frames outside 1..{VQM_MAX_BATCH}")
        pr = (ctypes.c_void_p * n)()
        pd = (ctypes.c_void_p * n)()
        keep = []  # the planes the pointers address, alive until the call returns
        w = h = None
        for i, (r, d) in enumerate(zip(refs, diss)):
            a, b, fw, fh, k = _pair(r, d, bpc)
            keep.append(k)
            if w is None:
                w, h = fw, fh
            elif (fw, fh) != (w, h):
                raise ValueError("frames of one batch must share their size")
            pr[i], pd[i] = a, b
        lw, lh = w >> (level - 1), h >> (level - 1)
        out_r = np.empty((n, lh, lw), np.float32)
        out_d = np.empty((n, lh, lw), np.float32)
        _check(lib().vqm_debug_pyramid_batch(self._h, pr, pd, n, w, h, int(bpc), int(level), out_r.ctypes.data,
                                             out_d.ctypes.data), "vqm_debug_pyramid_batch")
        return out_r, out_d


def vqm_ctx_create(device: int = 0, stream=None) -> Context:
    return Context(device, stream)


class FrameSet:
    """Plane pointers of many frame pairs, marshalled once for repeated
    vqm_score_frames calls (the planes stay referenced)."""

    def __init__(self, refs, diss, bpc: int):
        if len(refs) != len(diss) or not refs:
            raise ValueError("refs and dis must be non-empty and of equal length")
        n = len(refs)
        self.n, self.bpc = n, int(bpc)
        self.refs = (ctypes.c_void_p * n)()
        self.diss = (ctypes.c_void_p * n)()
        self._keep = []
        self.w = self.h = None
        for i, (r, d) in enumerate(zip(refs, diss)):
            a, b, w, h, k = _pair(r, d, bpc)
            if self.w is None:
                self.w, self.h = w, h
            elif (w, h) != (self.w, self.h):
                raise ValueError("all frames must share their size")
            self.refs[i], self.diss[i] = a, b
            self._keep.append(k)


def vqm_score_frames(ctxs, metric: int, frames: FrameSet, batch: int = VQM_MAX_BATCH, lag: int = 0,
                     want_lcs: bool = False, want_db: bool = False):
    """Score every frame of `frames` through the contexts `ctxs` (see the C
    call); returns the scores, followed by the 15 MS-SSIM level means per
    frame when want_lcs and the decibel forms when want_db."""
    handles = (ctypes.c_void_p * len(ctxs))(*[c._h.value for c in ctxs])
    scores = np.empty(frames.n, np.float64)
    lcs = np.empty((frames.n, VQM_MSSSIM_LCS), np.float64) if want_lcs else None
    db = np.empty(frames.n, np.float64) if want_db else None
    dp = ctypes.POINTER(ctypes.c_double)
    _check(lib().vqm_score_frames(handles, len(ctxs), int(metric), frames.refs, frames.diss, frames.n,
                                  frames.w, frames.h, frames.bpc, int(batch), int(lag),
                                  scores.ctypes.data_as(dp),
                                  lcs.ctypes.data_as(dp) if want_lcs else None,
                                  db.ctypes.data_as(dp) if want_db else None), "vqm_score_frames")
    out = (scores,) + ((lcs,) if want_lcs else ()) + ((db,) if want_db else ())
    return out if len(out) > 1 else scores


class Graph:
    """A ``vqm_graph``: one scoring pass over a fixed FrameSet of device
    frames, recorded once and replayed (see vqm_graph_create)."""

    def __init__(self, device: int, stream, metric: int, frames: FrameSet, batch: int = VQM_MAX_BATCH):
        self._h = ctypes.c_void_p()
        # the frames and the stream stay referenced for the graph's lifetime
        self.metric, self.frames, self._stream = int(metric), frames, stream
        _check(lib().vqm_graph_create(int(device), _stream_handle(stream), self.metric, frames.refs, frames.diss,
                                      frames.n, frames.w, frames.h, frames.bpc, int(batch), ctypes.byref(self._h)),
               "vqm_graph_create")

    def vqm_graph_launch(self):
        _check(lib().vqm_graph_launch(self._h), "vqm_graph_launch")

    def vqm_graph_collect(self, want_lcs: bool = False, want_db: bool = False):
        """The replay's scores, followed by the per-level means when want_lcs
        and the decibel forms when want_db."""
        n = self.frames.n
        scores = np.empty(n, np.float64)
        lcs = np.empty((n, VQM_MSSSIM_LCS), np.float64) if want_lcs else None
        db = np.empty(n, np.float64) if want_db else None
        dp = ctypes.POINTER(ctypes.c_double)
        _check(lib().vqm_graph_collect(self._h, scores.ctypes.data_as(dp),
                                       lcs.ctypes.data_as(dp) if want_lcs else None,
                                       db.ctypes.data_as(dp) if want_db else None), "vqm_graph_collect")
        out = (scores,) + ((lcs,) if want_lcs else ()) + ((db,) if want_db else ())
        return out if len(out) > 1 else scores

    def close(self):
        if self._h:
            lib().vqm_graph_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass
