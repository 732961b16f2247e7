"""Plain CPU oracle for the float_moment and float_psnr frame reductions.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never includes, links or calls it, and it imports nothing from the
HIP side.

The arithmetic lives in ``oracle.c`` (the loops the pages describe; see its
header for the page/section each step follows).  This module only builds
that file with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -O2, no fast-math, no contraction, default x86-64 (SSE2) code: float
# arithmetic in float, double in double, round to nearest even.
CFLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
          "-fPIC", "-shared", "-Wall", "-Wextra"]
LIBS = ["-lm"]

_lock = threading.Lock()
_lib = None


def build(out: str = LIB, mutant: int = 0) -> str:
    """Compile oracle.c into ``out``; ``mutant`` plants a test mistake."""
    cmd = ["gcc", *CFLAGS, f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", out, *LIBS]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    vp = ctypes.c_void_p
    i = ctypes.c_int
    pd = ctypes.c_ssize_t
    lib.oracle_fsq.argtypes = [ctypes.c_uint, i]
    lib.oracle_fsq.restype = ctypes.c_float
    for name in ("oracle_moment_sums", "oracle_moment_frame",
                 "oracle_psnr_noise"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, i, i, pd, i, dp]
        fn.restype = i
    lib.oracle_psnr_sum.argtypes = [vp, vp, i, i, pd, i, dp]
    lib.oracle_psnr_sum.restype = i
    lib.oracle_frames.argtypes = [vp, vp, i, i, pd, pd, i, i, dp, dp]
    lib.oracle_frames.restype = i
    lib.oracle_psnr_db.argtypes = [ctypes.c_double, i]
    lib.oracle_psnr_db.restype = ctypes.c_double
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB) or (
                    os.path.getmtime(LIB) < os.path.getmtime(SRC)):
                build()
            _lib = _bind(ctypes.CDLL(LIB))
        return _lib


class Oracle:
    """Thin marshalling wrapper; ``lib`` may be a mutant build."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    @staticmethod
    def _ptr(a: np.ndarray):
        assert a.flags["C_CONTIGUOUS"] or a.ndim <= 1
        return ctypes.c_void_p(a.ctypes.data)

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise ValueError(f"{what} returned {rc}")

    @staticmethod
    def _geom(plane: np.ndarray, w: int | None, stride: int | None):
        h, s = plane.shape[-2], plane.shape[-1]
        return (s if w is None else w), h, (s if stride is None else stride)

    def psnr_db(self, mse: float, bpc: int) -> float:
        """PSNR in dB from an MSE (a reading; parity unpinned)."""
        return float(self.lib.oracle_psnr_db(float(mse), int(bpc)))

    def fsq(self, x: int, bpc: int) -> float:
        return float(self.lib.oracle_fsq(int(x), int(bpc)))

    def moment_sums(self, ref, dis, bpc, w=None):
        w, h, stride = self._geom(ref, w, None)
        out = (ctypes.c_double * 4)()
        self._check(self.lib.oracle_moment_sums(
            self._ptr(ref), self._ptr(dis), w, h, stride, bpc, out),
            "oracle_moment_sums")
        return list(out)

    def moment_frame(self, ref, dis, bpc, w=None):
        w, h, stride = self._geom(ref, w, None)
        out = (ctypes.c_double * 4)()
        self._check(self.lib.oracle_moment_frame(
            self._ptr(ref), self._ptr(dis), w, h, stride, bpc, out),
            "oracle_moment_frame")
        return list(out)

    def psnr_sum(self, ref, dis, bpc, w=None):
        w, h, stride = self._geom(ref, w, None)
        out = ctypes.c_double()
        self._check(self.lib.oracle_psnr_sum(
            self._ptr(ref), self._ptr(dis), w, h, stride, bpc,
            ctypes.byref(out)), "oracle_psnr_sum")
        return out.value

    def psnr_noise(self, ref, dis, bpc, w=None):
        w, h, stride = self._geom(ref, w, None)
        out = (ctypes.c_double * 2)()
        self._check(self.lib.oracle_psnr_noise(
            self._ptr(ref), self._ptr(dis), w, h, stride, bpc, out),
            "oracle_psnr_noise")
        return list(out)

    def frames(self, ref, dis, bpc, w=None):
        """ref/dis: (F, h, stride) arrays.  Returns (moments[F,4], psnr[F,2])."""
        assert ref.shape == dis.shape and ref.ndim == 3
        f, h, stride = ref.shape
        return self.frames_flat(ref, dis, bpc, w=stride if w is None else w, h=h,
                                stride=stride, pitch=h * stride, nframes=f)

    def frames_flat(self, ref, dis, bpc, *, w, h, stride, pitch, nframes):
        """Frames laid out in one buffer each (any shape, C-contiguous):
        frame f starts ``f * pitch`` samples in, rows ``stride`` samples
        apart.  Returns (moments[F,4], psnr[F,2])."""
        assert ref.dtype == dis.dtype and ref.size == dis.size
        need = (nframes - 1) * pitch + (h - 1) * stride + w
        assert nframes >= 1 and ref.size >= need, (ref.size, need)
        mom = np.zeros((nframes, 4), np.float64)
        ps = np.zeros((nframes, 2), np.float64)
        dp = ctypes.POINTER(ctypes.c_double)
        self._check(self.lib.oracle_frames(
            self._ptr(ref), self._ptr(dis), w, h, stride, pitch, nframes, bpc,
            mom.ctypes.data_as(dp), ps.ctypes.data_as(dp)), "oracle_frames")
        return mom, ps
