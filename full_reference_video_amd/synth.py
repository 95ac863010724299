"""Seeded synthetic luma frames for the five scoring workloads.

This module is the one source of input frames for the tests, the benchmark and
the oracle's own tests. It holds none of the scoring arithmetic: it only draws
pixels. Every frame is a pure function of (config, frame index, size), so any
process can regenerate the exact bytes another process scored.

The pages measure on real clips (the Netflix 576x324 pair, Big Buck Bunny at
3840x2160, an 853x481 rescale, 1080p checkerboards; "Device-resident
ssimulacra2 and a single-wait MS-SSIM on SYCL", Sources, and "float_ssim_hip
decimates on the device", Consequences).  None of them is available here, so
these frames stand in for them with the same shapes, bit depths and frame
counts, and with content that has the usual mix of smooth structure and noise.

Recipe (fixed here so every run is reproducible):

* Field F, drawn once per config from ``default_rng(1000 * c)``:
  ``F(x, y) = 128 + 15 * sum_{k=1..4} sin(2*pi*(x cos t_k + y sin t_k)/P_k + p_k)``
  with ``P_k ~ U[24, 192)`` px, ``t_k ~ U[0, pi)``, ``p_k ~ U[0, 2*pi)``.  So
  ``|F - 128| <= 60``: amplitude 60 about an offset of 128.
* Per-frame noise from ``default_rng(1000 * c + 1 + t)`` for frame ``t``.
* Rounding with ``numpy.rint`` (ties to even), then clipping to
  ``[0, 2**bpc - 1]``.  Per-frame arithmetic is float32 (int16 uniform draws,
  float32 normal draws): the frames are inputs, not results, and only their
  exact bytes matter.

Configs (c = 1..5):

1. 576x324 8-bit, 1 frame: ref = F + U{-8..8}; dis = ref + N(0, 4^2).
2. 853x481 12-bit in uint16, 48 frames: ref = (F + U{-8..8}) * 4095/255;
   dis = 3x3 box blur of ref (symmetric edges, fp64) + N(0, 16^2).
3. 1920x1080 8-bit, 48 frames: a (w + 94)-wide canvas of F + U{-8..8}, frame
   t is columns [2t, 2t + w) (a pan of 2 px per frame); dis = 8*floor(ref/8)
   + N(0, 2^2) (banding plus noise).
4. 3840x2160 10-bit in uint16, 50 frames: ref = 4F + U{-16..16};
   dis = ref + N(0, 12^2).
5. 3840x2160 8-bit, 50 frames (MS-SSIM): ref = F + U{-8..8};
   dis = ref + N(0, 6^2).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one scoring workload."""

    index: int          # config number c, 1..5 (also the seed family)
    name: str
    metric: str         # "float_ssim" or "ms_ssim"
    w: int
    h: int
    bpc: int
    frames: int

    @property
    def dtype(self):
        return np.uint8 if self.bpc == 8 else np.uint16

    @property
    def frame_bytes(self) -> int:
        return self.w * self.h * np.dtype(self.dtype).itemsize


WORKLOADS = {
    1: Workload(1, "float_ssim_576x324_8bit", "float_ssim", 576, 324, 8, 1),
    2: Workload(2, "float_ssim_853x481_12bit", "float_ssim", 853, 481, 12, 48),
    3: Workload(3, "float_ssim_1920x1080_8bit", "float_ssim", 1920, 1080, 8, 48),
    4: Workload(4, "float_ssim_3840x2160_10bit", "float_ssim", 3840, 2160, 10, 50),
    5: Workload(5, "ms_ssim_3840x2160_8bit", "ms_ssim", 3840, 2160, 8, 50),
}

# Config 3 pans 2 px per frame over a canvas this much wider than the frame.
_PAN_STEP = 2
_PAN_EXTRA = 94


def _field_params(c: int):
    rng = np.random.default_rng(1000 * c)
    period = rng.uniform(24.0, 192.0, size=4)
    theta = rng.uniform(0.0, np.pi, size=4)
    phase = rng.uniform(0.0, 2.0 * np.pi, size=4)
    return rng, period, theta, phase


def sinusoid_field(c: int, w: int, h: int) -> np.ndarray:
    """Smooth field F of config ``c`` on a ``w`` x ``h`` grid, float64, 128 +- 60."""
    _, period, theta, phase = _field_params(c)
    x = np.arange(w, dtype=np.float64)[None, :]
    y = np.arange(h, dtype=np.float64)[:, None]
    f = np.zeros((h, w), dtype=np.float64)
    for k in range(4):
        # The phase is separable in x and y; sin(a + b) needs only 1-D tables.
        ax = 2.0 * np.pi * x * np.cos(theta[k]) / period[k] + phase[k]
        ay = 2.0 * np.pi * y * np.sin(theta[k]) / period[k]
        f += np.sin(ax) * np.cos(ay) + np.cos(ax) * np.sin(ay)
    return 128.0 + 15.0 * f


def _quantise(a: np.ndarray, bpc: int) -> np.ndarray:
    hi = (1 << bpc) - 1
    out = np.clip(np.rint(a), 0, hi)
    return out.astype(np.uint8 if bpc == 8 else np.uint16)


def _box3_symmetric(a: np.ndarray) -> np.ndarray:
    p = np.pad(a.astype(np.float64), 1, mode="symmetric")
    h, w = a.shape
    acc = np.zeros((h, w), dtype=np.float64)
    for dy in range(3):
        for dx in range(3):
            acc += p[dy:dy + h, dx:dx + w]
    return acc / 9.0


class FrameSource:
    """Deterministic frame pairs of one workload, optionally at another size.

    ``w``/``h`` override the workload's size (tests use smaller frames with the
    same recipe); the field and the noise streams do not depend on the size
    beyond the grid they are drawn on.
    """

    def __init__(self, c: int, w: int | None = None, h: int | None = None,
                 bpc: int | None = None):
        wl = WORKLOADS[c]
        self.c = c
        self.workload = wl
        self.w = wl.w if w is None else int(w)
        self.h = wl.h if h is None else int(h)
        self.bpc = wl.bpc if bpc is None else int(bpc)
        if c == 3:
            canvas_w = self.w + _PAN_EXTRA
            rng, _, _, _ = _field_params(c)
            f = sinusoid_field(c, canvas_w, self.h)
            # Canvas noise comes after the field parameters in the same stream.
            noise = rng.integers(-8, 9, size=f.shape, dtype=np.int16)
            self._canvas = _quantise((f + noise) * ((1 << self.bpc) - 1) / 255.0, self.bpc)
            self._field = None
        else:
            self._canvas = None
            self._field = sinusoid_field(c, self.w, self.h).astype(np.float32)

    @property
    def dtype(self):
        return np.uint8 if self.bpc == 8 else np.uint16

    def pair(self, t: int):
        """Return (ref, dis) for frame ``t`` as C-contiguous uint8/uint16 arrays."""
        c, bpc = self.c, self.bpc
        rng = np.random.default_rng(1000 * c + 1 + t)
        full = (1 << bpc) - 1
        shape = (self.h, self.w)

        def uniform(k):
            return rng.integers(-k, k + 1, size=shape, dtype=np.int16).astype(np.float32)

        def gauss(sigma):
            return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)

        if c == 1 or c == 5:
            ref = _quantise((self._field + uniform(8)) * np.float32(full / 255.0), bpc)
            sigma = 4.0 if c == 1 else 6.0
            dis = _quantise(ref + gauss(sigma * full / 255.0), bpc)
        elif c == 2:
            ref = _quantise((self._field + uniform(8)) * np.float32(full / 255.0), bpc)
            dis = _quantise(_box3_symmetric(ref) + gauss(16.0 * full / 4095.0), bpc)
        elif c == 3:
            x0 = (_PAN_STEP * t) % (_PAN_EXTRA + 1)
            ref = np.ascontiguousarray(self._canvas[:, x0:x0 + self.w])
            step = 8 * ((full + 1) // 256)
            band = ((ref // step) * step).astype(np.float32)
            dis = _quantise(band + gauss(2.0 * (full + 1) / 256.0), bpc)
        elif c == 4:
            scale = np.float32((full + 1) / 1024.0)
            ref = _quantise((np.float32(4.0) * self._field + uniform(16)) * scale, bpc)
            dis = _quantise(ref + gauss(12.0 * scale), bpc)
        else:
            raise ValueError(f"unknown config {c}")
        return np.ascontiguousarray(ref), np.ascontiguousarray(dis)


def chroma_pair(c: int, t: int, plane: int, w: int, h: int, bpc: int):
    """(ref, dis) of chroma plane 1 (Cb) or 2 (Cr), w x h, of frame ``t`` in
    the style of config ``c``: a smooth field of its own (seed
    1000 c + 100 plane), narrower than luma about the mid value, plus uniform
    noise in +-4; dis adds Gaussian noise of sigma 3 (8-bit units)."""
    full = (1 << bpc) - 1
    rng = np.random.default_rng(1000 * c + 100 * plane)
    period = rng.uniform(24.0, 192.0, size=3)
    theta = rng.uniform(0.0, np.pi, size=3)
    phase = rng.uniform(0.0, 2.0 * np.pi, size=3)
    x = np.arange(w, dtype=np.float64)[None, :]
    y = np.arange(h, dtype=np.float64)[:, None]
    f = np.full((h, w), 128.0)
    for k in range(3):
        f = f + 10.0 * np.sin(2.0 * np.pi * (x * np.cos(theta[k]) + y * np.sin(theta[k])) / period[k] + phase[k])
    noise = np.random.default_rng(1000 * c + 100 * plane + 1 + t)
    scale = full / 255.0
    ref = _quantise((f + noise.integers(-4, 5, size=(h, w))) * scale, bpc)
    dis = _quantise(ref + noise.standard_normal(size=(h, w)) * (3.0 * scale), bpc)
    return np.ascontiguousarray(ref), np.ascontiguousarray(dis)


def random_planes(seed: int, w: int, h: int, bpc: int, kind: str = "uniform"):
    """Small seeded planes for edge-case and property tests.

    ``kind``: "uniform" draws every sample in [0, 2**bpc - 1]; "max" fills with
    the largest sample; "zero" with zeros; "checker" a +-1-level checkerboard
    about mid-range.
    """
    rng = np.random.default_rng(seed)
    hi = (1 << bpc) - 1
    dt = np.uint8 if bpc == 8 else np.uint16
    if kind == "uniform":
        return rng.integers(0, hi + 1, size=(h, w)).astype(dt)
    if kind == "max":
        return np.full((h, w), hi, dtype=dt)
    if kind == "zero":
        return np.zeros((h, w), dtype=dt)
    if kind == "checker":
        yy, xx = np.mgrid[0:h, 0:w]
        return ((hi + 1) // 2 + ((xx + yy) & 1)).astype(dt)
    raise ValueError(kind)


def _box5_symmetric(a: np.ndarray) -> np.ndarray:
    """5 x 5 mean with half-sample symmetric edges, in fp64 (input
    preparation only)."""
    p = np.pad(a, 2, mode="symmetric")
    h, w = a.shape
    acc = np.zeros((h, w), dtype=np.float64)
    for dy in range(5):
        for dx in range(5):
            acc += p[dy:dy + h, dx:dx + w]
    return acc / 25.0


def ss2_images(seed: int, w: int, h: int, channels: int = 3):
    """The two pictures' colour-transformed planes for the ssimulacra2
    per-scale chain: lists ``ref``, ``dis`` of ``channels`` float32 h x w
    planes.

    The pages measure ssimulacra2 on the Netflix 576x324 pair, Big Buck Bunny
    at 3840x2160 and an 853x481 rescale ("Device-resident ssimulacra2 and a
    single-wait MS-SSIM on SYCL", Sources and Finding 5); none is available
    here, so seeded planes of those sizes stand in.  Each reference channel
    is a smooth field in [0, 1] (3 sinusoids of amplitude 0.08 about a level
    drawn in [0.3, 0.7], from ``default_rng(seed * 10 + channel)``) plus
    uniform noise in +-0.02; the distorted channel adds Gaussian noise of
    sigma 0.01, clipped to [0, 1].
    """
    refs, diss = [], []
    x = np.arange(w, dtype=np.float64)[None, :]
    y = np.arange(h, dtype=np.float64)[:, None]
    for ch in range(channels):
        rng = np.random.default_rng(seed * 10 + ch)
        level = rng.uniform(0.3, 0.7)
        f = np.full((h, w), level)
        for _ in range(3):
            period = rng.uniform(12.0, 96.0)
            theta = rng.uniform(0.0, np.pi)
            phase = rng.uniform(0.0, 2.0 * np.pi)
            f = f + 0.08 * np.sin(2.0 * np.pi * (x * np.cos(theta) + y * np.sin(theta)) / period + phase)
        img1 = np.clip(f + rng.uniform(-0.02, 0.02, size=(h, w)), 0.0, 1.0).astype(np.float32)
        img2 = np.clip(img1 + rng.normal(0.0, 0.01, size=(h, w)), 0.0, 1.0).astype(np.float32)
        refs.append(img1)
        diss.append(img2)
    return refs, diss


def ss2_planes(seed: int, w: int, h: int, channels: int = 3):
    """Inputs of the ssimulacra2 per-scale statistics: per channel the seven
    float32 planes (img1, img2, mu1, mu2, s11, s22, s12), each h x w.

    img1 and img2 are ``ss2_images(seed, w, h, channels)``.  The blurred
    planes are 5 x 5 means (symmetric edges, fp64, then
    rounded to float32) of the images and of their products: a stand-in for
    the metric's own blur, so that every variance the statistics form is
    non-negative, as a blur with non-negative weights keeps it.
    """
    out = []
    refs, diss = ss2_images(seed, w, h, channels)
    for img1, img2 in zip(refs, diss):
        a, b = img1.astype(np.float64), img2.astype(np.float64)
        mu1, mu2 = _box5_symmetric(a), _box5_symmetric(b)
        s11, s22, s12 = _box5_symmetric(a * a), _box5_symmetric(b * b), _box5_symmetric(a * b)
        out.append([np.ascontiguousarray(p, dtype=np.float32) for p in (img1, img2, mu1, mu2, s11, s22, s12)])
    return out
