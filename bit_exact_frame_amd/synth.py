"""Seeded synthetic luma planes for the frame workloads.

This module only draws samples.  It holds none of the reductions'
arithmetic (no squares, no sums), so the CPU oracle and the HIP path can
both take their inputs from it.

Every plane is drawn by ``numpy.random.Generator(PCG64(SeedSequence(
[SEED, workload, frame])))``: the reference plane first, then the distorted
one.  Planes are C-ordered ``(h, stride)``; samples beyond ``w`` in each row
are padding, filled with the container's all-ones value so that a kernel
that reads them gives a wrong answer.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED = 0xBEF


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    bpc: int
    w: int
    h: int
    stride: int
    frames: int
    recipe: str

    @property
    def dtype(self):
        return np.uint8 if self.bpc == 8 else np.uint16

    @property
    def sample_bytes(self) -> int:
        return 1 if self.bpc == 8 else 2

    @property
    def bytes_per_frame(self) -> int:
        """Algorithmic bytes: each of the two planes' w*h samples read once."""
        return 2 * self.w * self.h * self.sample_bytes


WORKLOADS = {
    1: Workload(1, "8bit_176x144_uniform", 8, 176, 144, 176, 4,
                "ref, dis i.i.d. uniform [0,255]"),
    2: Workload(2, "10bit_1920x1080_lowbits_noise8", 10, 1920, 1080, 1920,
                32, "ref = 4*U[0,255] + U[1,3]; dis = clip(ref + rint(N(0,8^2)), 0, 1023)"),
    3: Workload(3, "12bit_2560x1440_stride2624_noise64", 12, 2560, 1440,
                2624, 32, "ref U[0,4095]; dis = clip(ref + rint(N(0,64^2)), 0, 4095)"),
    4: Workload(4, "16bit_3840x2160_fullrange", 16, 3840, 2160, 3840, 16,
                "ref, dis i.i.d. uniform [0,65535]"),
    5: Workload(5, "16bit_3840x2160_halfrange", 16, 3840, 2160, 3840, 8,
                "ref U[32768,65535], dis U[0,32767]"),
    # larger frames and real-content statistics (measured like the five above)
    6: Workload(6, "16bit_7680x4320_fullrange", 16, 7680, 4320, 7680, 4,
                "ref, dis i.i.d. uniform [0,65535] (sums pass 2^55)"),
    7: Workload(7, "16bit_4096x2560_nearmax_small5", 16, 4096, 2560, 4096, 4,
                "near-maximum content: ref U[60000,65535], dis U[58000,65535], one sample "
                "in twenty of each replaced by U[0,8191] (both planes pass 2^55, with ties "
                "there)"),
    8: Workload(8, "16bit_3840x2160_widened_dither", 16, 3840, 2160, 3840, 16,
                "smooth 8-bit content widened to 16 bits with a seeded low byte "
                "(widened_frames, mode dither)"),
}


def rng_for(key: int, frame: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([SEED, int(key), int(frame)])))


def _draw(wl: Workload, rng: np.random.Generator):
    h, w = wl.h, wl.w
    if wl.key == 1:
        ref = rng.integers(0, 256, size=(h, w))
        dis = rng.integers(0, 256, size=(h, w))
    elif wl.key == 2:
        # "low two bits forced non-zero": the 2-bit field is drawn from
        # {1, 2, 3}, so every codeword has a fractional part at 10 bpc.
        ref = 4 * rng.integers(0, 256, size=(h, w)) + rng.integers(1, 4, size=(h, w))
        dis = np.clip(ref + np.rint(rng.normal(0.0, 8.0, size=(h, w))), 0, 1023)
    elif wl.key == 3:
        ref = rng.integers(0, 4096, size=(h, w))
        dis = np.clip(ref + np.rint(rng.normal(0.0, 64.0, size=(h, w))), 0, 4095)
    elif wl.key == 4:
        ref = rng.integers(0, 65536, size=(h, w))
        dis = rng.integers(0, 65536, size=(h, w))
    elif wl.key == 5:
        ref = rng.integers(32768, 65536, size=(h, w))
        dis = rng.integers(0, 32768, size=(h, w))
    elif wl.key == 6:
        ref = rng.integers(0, 65536, size=(h, w))
        dis = rng.integers(0, 65536, size=(h, w))
    elif wl.key == 7:
        ref = nearmax_plane(rng, h, w, 60000)
        dis = nearmax_plane(rng, h, w, 58000)
    else:
        raise KeyError(wl.key)
    return ref, dis


def make_frames(key: int, frames: int | None = None, first: int = 0):
    """Return (ref, dis): arrays of shape (F, h, stride) of the workload's
    container dtype, frames ``first .. first+F-1``."""
    wl = WORKLOADS[key]
    n = wl.frames if frames is None else int(frames)
    if key == 8:
        return widened_frames("dither", n)
    pad = np.iinfo(wl.dtype).max
    ref = np.full((n, wl.h, wl.stride), pad, dtype=wl.dtype)
    dis = np.full((n, wl.h, wl.stride), pad, dtype=wl.dtype)
    for k in range(n):
        r, d = _draw(wl, rng_for(key, first + k))
        ref[k, :, :wl.w] = r
        dis[k, :, :wl.w] = d
    return ref, dis


def nearmax_plane(rng: np.random.Generator, h: int, w: int, lo: int,
                  small: float = 0.05) -> np.ndarray:
    """A 16-bit plane of near-maximum content: U[lo, 65535], with a fraction
    ``small`` of the samples replaced by U[0, 8191].  At 4096x2560 and lo of
    58000 or more the plane's sum of float squares passes 2^55 units in its
    last rows; the small codewords' squares are the terms with bits below
    the last place of that binade, some of them ties."""
    x = rng.integers(lo, 65536, size=(h, w))
    m = rng.random(size=(h, w)) < small
    x[m] = rng.integers(0, 8192, size=int(m.sum()))
    return x


def uniform_planes(seed: int, frames: int, h: int, w: int, stride: int,
                   bpc: int, lo: int = 0, hi: int | None = None):
    """Generic seeded uniform planes for parity cases of arbitrary shape."""
    dtype = np.uint8 if bpc == 8 else np.uint16
    top = (1 << (8 if bpc == 8 else 16)) if hi is None else hi
    pad = np.iinfo(dtype).max
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, 99, seed])))
    ref = np.full((frames, h, stride), pad, dtype=dtype)
    dis = np.full((frames, h, stride), pad, dtype=dtype)
    ref[:, :, :w] = rng.integers(lo, top, size=(frames, h, w))
    dis[:, :, :w] = rng.integers(lo, top, size=(frames, h, w))
    return ref, dis


# ---------------------------------------------------------------------------
# Smooth 8-bit content widened to 16 bits (stand-in for real footage widened
# three ways: ADR-1497, Consequences).  The 8-bit picture is a seeded sum of
# a few low-frequency waves and a gradient, plus a little noise, with a
# brightness that steps by frame so that the widened frames' second-moment
# sums fall on both sides of 2^53 units, and a dark band in the bottom rows
# (small codewords: odd float squares once the sum is past 2^53); the
# distorted picture is the same scene shifted by one pixel with its own
# noise.  Widening: "shift" x << 8, "x257" x * 257 (full range), "dither"
# x << 8 plus a seeded uniform low byte.

WIDEN_MODES = ("shift", "x257", "dither")


def smooth_8bit(seed: int, h: int, w: int, shift: int = 0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, 313, seed])))
    yy, xx = np.mgrid[0:h, 0:w].astype(np.float64)
    xx = xx + shift
    img = 40.0 + 30.0 * (seed // 2 % 4) + 120.0 * (xx / w) * (1.0 - 0.5 * yy / h)
    for _ in range(4):
        fx, fy = rng.uniform(0.5, 6.0, size=2)
        ph = rng.uniform(0, 2 * np.pi)
        amp = rng.uniform(10.0, 35.0)
        img += amp * np.sin(2 * np.pi * (fx * xx / w + fy * yy / h) + ph)
    img += rng.normal(0.0, 2.0, size=(h, w))
    img[int(0.85 * h):] *= 0.06  # a dark band at the bottom (codewords below 16)
    return np.clip(np.rint(img), 0, 255).astype(np.int64)


def widened_frames(mode: str, frames: int, h: int = 2160, w: int = 3840):
    """(ref, dis) uint16 arrays (frames, h, w) of smooth content widened by
    ``mode`` (one of WIDEN_MODES)."""
    if mode not in WIDEN_MODES:
        raise KeyError(mode)
    ref = np.empty((frames, h, w), np.uint16)
    dis = np.empty((frames, h, w), np.uint16)
    for k in range(frames):
        r8 = smooth_8bit(2 * k, h, w)
        d8 = smooth_8bit(2 * k + 1, h, w, shift=1)
        if mode == "shift":
            r, d = r8 << 8, d8 << 8
        elif mode == "x257":
            r, d = r8 * 257, d8 * 257
        else:
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, 314, k])))
            r = (r8 << 8) | rng.integers(0, 256, size=(h, w))
            d = (d8 << 8) | rng.integers(0, 256, size=(h, w))
        ref[k], dis[k] = r, d
    return ref, dis


def yuv420_frames(seed: int, frames: int, w: int, h: int, bpc: int, pad: int = 0,
                  lo: int = 0, hi: int | None = None, noise: float | None = None):
    """Seeded 4:2:0 pictures: a luma plane of w x h and two chroma planes of
    ceil(w/2) x ceil(h/2), each row padded by ``pad`` samples of the
    container's top value.  ref is uniform [lo, hi); dis is independent
    uniform, or ref plus rint(N(0, noise^2)) clipped to [0, 2^bpc - 1] when
    ``noise`` is given.  Returns [(ref, dis)] per plane, arrays (F, h_p, w_p + pad)."""
    dtype = np.uint8 if bpc == 8 else np.uint16
    top = np.iinfo(dtype).max
    hi = (1 << bpc) if hi is None else hi
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, 420, seed])))
    out = []
    for (pw, ph) in ((w, h), ((w + 1) // 2, (h + 1) // 2), ((w + 1) // 2, (h + 1) // 2)):
        ref = np.full((frames, ph, pw + pad), top, dtype=dtype)
        dis = np.full((frames, ph, pw + pad), top, dtype=dtype)
        r = rng.integers(lo, hi, size=(frames, ph, pw))
        if noise is None:
            d = rng.integers(lo, hi, size=(frames, ph, pw))
        else:
            d = np.clip(r + np.rint(rng.normal(0.0, noise, size=r.shape)), 0, (1 << bpc) - 1)
        ref[:, :, :pw] = r
        dis[:, :, :pw] = d
        out.append((ref, dis))
    return out

