"""Python view of the plain C oracle (``vqm_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle is the yardstick the HIP library is held
against; only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg may import this package.  It shares no code with the HIP path.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vqm_oracle.c")
_SS2_SRC = os.path.join(_HERE, "ss2_oracle.c")
SOURCES = [_SRC, _SS2_SRC]
_LIB = os.path.join(_HERE, "libvqm_oracle.so")

# Contraction off and no fast-math: every fp32 product and the single
# rounding of each decimated sample must be what the C source says.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(cc: str = "gcc") -> str:
    """Compile the oracle into ``oracle/libvqm_oracle.so`` (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run([cc, *CFLAGS, "-o", tmp, *SOURCES, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Load the oracle library, building it first if it is absent.

    ``VQM_ORACLE_LIB`` names another build of the same source to load instead
    (the mutation test points it at deliberately broken copies).
    """
    global _lib
    if _lib is None:
        path = os.environ.get("VQM_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f) for f in SOURCES):
                build()
        L = ctypes.CDLL(path)
        vp, ip, fp, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
        L.vqm_oracle_scale.argtypes = [ip, ip]
        L.vqm_oracle_scale.restype = ip
        L.vqm_oracle_tap.argtypes = [ip]
        L.vqm_oracle_tap.restype = ctypes.c_float
        L.vqm_oracle_decimated_dim.argtypes = [ip, ip]
        L.vqm_oracle_decimated_dim.restype = ip
        L.vqm_oracle_sample_plane.argtypes = [vp, ip, ip, ip, fp]
        L.vqm_oracle_decimate.argtypes = [vp, ip, ip, ip, ip, fp]
        L.vqm_oracle_ssim_planes.argtypes = [fp, fp, ip, ip, dp, dp]
        L.vqm_oracle_ssim.argtypes = [vp, vp, ip, ip, ip, dp]
        L.vqm_oracle_msssim_level_maps.argtypes = [fp, fp, ip, ip, dp, dp, dp]
        L.vqm_oracle_downsample.argtypes = [fp, ip, ip, fp]
        L.vqm_oracle_msssim.argtypes = [vp, vp, ip, ip, ip, dp, dp]
        L.vqm_oracle_plane_dims.argtypes = [ip, ip, ip, ip, ctypes.POINTER(ip), ctypes.POINTER(ip)]
        L.vqm_oracle_plane_dims.restype = ip
        L.vqm_oracle_db.argtypes = [ctypes.c_double]
        L.vqm_oracle_db.restype = ctypes.c_double
        L.vqm_oracle_ss2_channel_sums.argtypes = [fp] * 7 + [ip, ip, dp]
        L.vqm_oracle_ss2_channel_sums.restype = ip
        fl = ctypes.c_float
        for name in ("vqm_oracle_two_sum", "vqm_oracle_two_prod"):
            getattr(L, name).argtypes = [fl, fl, fp]
            getattr(L, name).restype = None
        for name in ("vqm_oracle_ff_add", "vqm_oracle_ff_mul", "vqm_oracle_ff_div"):
            getattr(L, name).argtypes = [fp, fp, fp]
            getattr(L, name).restype = None
        L.vqm_oracle_iir_line.argtypes = [fp, ip, fp, fp]
        L.vqm_oracle_ss2_blur.argtypes = [fp, ip, ip, fp, fp]
        L.vqm_oracle_ss2_downsampled_dim.argtypes = [ip, ip, ctypes.POINTER(ip), ctypes.POINTER(ip)]
        L.vqm_oracle_ss2_downsampled_dim.restype = None
        L.vqm_oracle_ss2_downsample.argtypes = [fp, ip, ip, fp]
        L.vqm_oracle_ss2_cascade_coefficients.argtypes = [ctypes.c_double, fp]
        L.vqm_oracle_ss2_chain.argtypes = [vp, vp, ip, ip, ip, ip, fp, dp]
        for name in ("vqm_oracle_iir_line", "vqm_oracle_ss2_blur", "vqm_oracle_ss2_downsample",
                     "vqm_oracle_ss2_cascade_coefficients", "vqm_oracle_ss2_chain"):
            getattr(L, name).restype = ip
        L.vqm_oracle_msssim_combine.argtypes = [dp]
        L.vqm_oracle_msssim_combine.restype = ctypes.c_double
        for name in ("vqm_oracle_sample_plane", "vqm_oracle_decimate", "vqm_oracle_ssim_planes",
                     "vqm_oracle_ssim", "vqm_oracle_msssim_level_maps", "vqm_oracle_downsample",
                     "vqm_oracle_msssim"):
            getattr(L, name).restype = ip
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what} failed with {rc} ({os.strerror(-rc) if rc < 0 else rc})")
        self.rc = rc


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _raw(a, bpc):
    dt = np.uint8 if bpc == 8 else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != dt:
        raise TypeError(f"bpc {bpc} needs {np.dtype(dt).name} samples, got {a.dtype}")
    return a


def _check(rc, what):
    if rc != 0:
        raise OracleError(rc, what)


def scale(w: int, h: int) -> int:
    return lib().vqm_oracle_scale(int(w), int(h))


def tap(s: int) -> np.float32:
    return np.float32(lib().vqm_oracle_tap(int(s)))


def decimated_dim(n: int, s: int) -> int:
    return lib().vqm_oracle_decimated_dim(int(n), int(s))


def sample_plane(raw: np.ndarray, bpc: int) -> np.ndarray:
    raw = _raw(raw, bpc)
    h, w = raw.shape
    out = np.empty((h, w), np.float32)
    _check(lib().vqm_oracle_sample_plane(_ptr(raw), w, h, bpc, _ptr(out)), "sample_plane")
    return out


def decimate(raw: np.ndarray, bpc: int, s: int) -> np.ndarray:
    raw = _raw(raw, bpc)
    h, w = raw.shape
    out = np.empty((decimated_dim(h, s), decimated_dim(w, s)), np.float32)
    _check(lib().vqm_oracle_decimate(_ptr(raw), w, h, bpc, int(s), _ptr(out)), "decimate")
    return out


def ssim_planes(ref: np.ndarray, dis: np.ndarray, want_map: bool = False):
    ref = np.ascontiguousarray(ref, np.float32)
    dis = np.ascontiguousarray(dis, np.float32)
    h, w = ref.shape
    score = ctypes.c_double()
    m = np.empty((max(h - 10, 0), max(w - 10, 0)), np.float64) if want_map else None
    _check(lib().vqm_oracle_ssim_planes(_ptr(ref), _ptr(dis), w, h, ctypes.byref(score),
                                        _ptr(m) if want_map else None), "ssim_planes")
    return (score.value, m) if want_map else score.value


def ssim(ref: np.ndarray, dis: np.ndarray, bpc: int) -> float:
    ref, dis = _raw(ref, bpc), _raw(dis, bpc)
    h, w = ref.shape
    score = ctypes.c_double()
    _check(lib().vqm_oracle_ssim(_ptr(ref), _ptr(dis), w, h, bpc, ctypes.byref(score)), "ssim")
    return score.value


def ssim_rc(ref: np.ndarray, dis: np.ndarray, w: int, h: int, bpc: int) -> int:
    """Return code of the oracle's float_ssim for the given (possibly bad) arguments."""
    score = ctypes.c_double()
    return lib().vqm_oracle_ssim(_ptr(ref), _ptr(dis), w, h, bpc, ctypes.byref(score))


def msssim_level_maps(ref: np.ndarray, dis: np.ndarray):
    ref = np.ascontiguousarray(ref, np.float32)
    dis = np.ascontiguousarray(dis, np.float32)
    h, w = ref.shape
    shp = (h - 10, w - 10)
    l, c, s = (np.empty(shp, np.float64) for _ in range(3))
    _check(lib().vqm_oracle_msssim_level_maps(_ptr(ref), _ptr(dis), w, h, _ptr(l), _ptr(c),
                                              _ptr(s)), "msssim_level_maps")
    return l, c, s


def downsample(plane: np.ndarray) -> np.ndarray:
    plane = np.ascontiguousarray(plane, np.float32)
    h, w = plane.shape
    out = np.empty((h // 2, w // 2), np.float32)
    _check(lib().vqm_oracle_downsample(_ptr(plane), w, h, _ptr(out)), "downsample")
    return out


def msssim(ref: np.ndarray, dis: np.ndarray, bpc: int, want_lcs: bool = False):
    ref, dis = _raw(ref, bpc), _raw(dis, bpc)
    h, w = ref.shape
    score = ctypes.c_double()
    lcs = np.empty(15, np.float64)
    _check(lib().vqm_oracle_msssim(_ptr(ref), _ptr(dis), w, h, bpc, ctypes.byref(score),
                                   _ptr(lcs)), "msssim")
    return (score.value, lcs) if want_lcs else score.value


def msssim_combine(lcs) -> float:
    """MS-SSIM of 15 level means L_1..L_5, C_1..C_5, S_1..S_5 (the oracle's combine)."""
    a = np.ascontiguousarray(lcs, np.float64)
    if a.shape != (15,):
        raise ValueError(f"15 level means expected, got shape {a.shape}")
    return lib().vqm_oracle_msssim_combine(_ptr(a))


def msssim_rc(ref: np.ndarray, dis: np.ndarray, w: int, h: int, bpc: int) -> int:
    score = ctypes.c_double()
    return lib().vqm_oracle_msssim(_ptr(ref), _ptr(dis), w, h, bpc, ctypes.byref(score), None)


def db(ssim: float) -> float:
    """-10 log10(1 - ssim), +inf at ssim >= 1 ([ADR-1405] Consequences, enable_db)."""
    return lib().vqm_oracle_db(float(ssim))


CHROMA_420, CHROMA_422, CHROMA_444 = 0, 1, 2


def plane_dims(w: int, h: int, chroma: int, plane: int):
    """(width, height) of plane 0..2 of a w x h picture in a chroma layout."""
    pw, ph = ctypes.c_int(), ctypes.c_int()
    _check(lib().vqm_oracle_plane_dims(w, h, chroma, plane, ctypes.byref(pw), ctypes.byref(ph)), "plane_dims")
    return pw.value, ph.value


# ---------------------------------------------------------------- ssimulacra2

SS2_PLANES = ("img1", "img2", "mu1", "mu2", "s11", "s22", "s12")


def ss2_channel_sums(img1, img2, mu1, mu2, s11, s22, s12) -> np.ndarray:
    """The six ssimulacra2 sums of one channel at one scale (fp64, in the
    order sum d, sum d^4, sum art, sum art^4, sum det, sum det^4)."""
    planes = [np.ascontiguousarray(p, np.float32) for p in (img1, img2, mu1, mu2, s11, s22, s12)]
    h, w = planes[0].shape
    for p in planes:
        if p.shape != (h, w):
            raise ValueError("all seven planes must have one shape")
    out = np.empty(6, np.float64)
    _check(lib().vqm_oracle_ss2_channel_sums(*[_ptr(p) for p in planes], w, h, _ptr(out)), "ss2_channel_sums")
    return out


def _pair_out(fn, *args):
    out = np.empty(2, np.float32)
    fn(*args, _ptr(out))
    return out[0], out[1]


def two_sum(a, b):
    return _pair_out(lib().vqm_oracle_two_sum, float(np.float32(a)), float(np.float32(b)))


def two_prod(a, b):
    return _pair_out(lib().vqm_oracle_two_prod, float(np.float32(a)), float(np.float32(b)))


def _ff(name, a, b):
    pa = np.ascontiguousarray(a, np.float32)
    pb = np.ascontiguousarray(b, np.float32)
    if pa.shape != (2,) or pb.shape != (2,):
        raise ValueError("pairs are two float32 values (hi, lo)")
    return _pair_out(getattr(lib(), name), _ptr(pa), _ptr(pb))


def ff_add(a, b):
    return _ff("vqm_oracle_ff_add", a, b)


def ff_mul(a, b):
    return _ff("vqm_oracle_ff_mul", a, b)


def ff_div(a, b):
    return _ff("vqm_oracle_ff_div", a, b)


# ------------------------------------------------- ssimulacra2 per-scale chain


def _coef(coef) -> np.ndarray:
    c = np.ascontiguousarray(coef, np.float32)
    if c.shape != (4,):
        raise ValueError("the recursion takes four coefficients (B, a1, a2, a3)")
    return c


def ss2_cascade_coefficients(sigma: float) -> np.ndarray:
    """(B, a1, a2, a3) of three symmetric exponential smoothers whose impulse
    response has variance sigma^2, as float32."""
    out = np.empty(4, np.float32)
    _check(lib().vqm_oracle_ss2_cascade_coefficients(float(sigma), _ptr(out)), "ss2_cascade_coefficients")
    return out


def iir_line(x, coef) -> np.ndarray:
    """One line through the causal, then anticausal, third-order recursion."""
    x = np.ascontiguousarray(x, np.float32)
    c = _coef(coef)
    y = np.empty_like(x)
    _check(lib().vqm_oracle_iir_line(_ptr(x), x.size, _ptr(c), _ptr(y)), "iir_line")
    return y


def ss2_blur(plane, coef) -> np.ndarray:
    """The recursion along every row, then every column."""
    plane = np.ascontiguousarray(plane, np.float32)
    h, w = plane.shape
    c = _coef(coef)
    out = np.empty_like(plane)
    _check(lib().vqm_oracle_ss2_blur(_ptr(plane), w, h, _ptr(c), _ptr(out)), "ss2_blur")
    return out


def ss2_downsampled_dim(w: int, h: int):
    ow, oh = ctypes.c_int(), ctypes.c_int()
    lib().vqm_oracle_ss2_downsampled_dim(int(w), int(h), ctypes.byref(ow), ctypes.byref(oh))
    return ow.value, oh.value


def ss2_downsample(plane) -> np.ndarray:
    plane = np.ascontiguousarray(plane, np.float32)
    h, w = plane.shape
    ow, oh = ss2_downsampled_dim(w, h)
    out = np.empty((oh, ow), np.float32)
    _check(lib().vqm_oracle_ss2_downsample(_ptr(plane), w, h, _ptr(out)), "ss2_downsample")
    return out


def ss2_chain(ref_planes, dis_planes, nscales: int, coef) -> np.ndarray:
    """The six sums per channel at every scale, shape [nscales, nch, 6]."""
    ref = [np.ascontiguousarray(p, np.float32) for p in ref_planes]
    dis = [np.ascontiguousarray(p, np.float32) for p in dis_planes]
    if len(ref) != len(dis) or not ref:
        raise ValueError("one reference and one distorted plane per channel")
    h, w = ref[0].shape
    for p in ref + dis:
        if p.shape != (h, w):
            raise ValueError("all planes must have one shape")
    nch = len(ref)
    arr = ctypes.c_void_p * nch
    rp = arr(*[p.ctypes.data for p in ref])
    dp_ = arr(*[p.ctypes.data for p in dis])
    c = _coef(coef)
    out = np.empty((max(int(nscales), 1), nch, 6), np.float64)
    _check(lib().vqm_oracle_ss2_chain(rp, dp_, nch, w, h, int(nscales), _ptr(c), _ptr(out)), "ss2_chain")
    return out
