"""ctypes binding of the host emulation library (tests only).

The emulation (bit_exact_frame_amd/csrc/host_emu.cpp, entry points declared
in host_emu.h) runs the kernels' steps serially on host planes with the
same step header.  It is not part of libbef.so: this module builds it with
g++ into a temporary directory once per process (or loads a given build, such
as one with a planted break) and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import tempfile
import threading

import numpy as np

from bit_exact_frame_amd import build as _build

_vp, _i, _pd, _u = ctypes.c_void_p, ctypes.c_int, ctypes.c_ssize_t, ctypes.c_uint
_u64p = ctypes.POINTER(ctypes.c_uint64)

_lock = threading.Lock()
_default = None

HEADER = os.path.join(_build.CSRC, "host_emu.h")


def _bind(lib):
    lib.bef_host_plane_units.argtypes = [_vp, _i, _i, _pd, _i, _u, _u64p]
    lib.bef_host_noise_units.argtypes = [_vp, _vp, _i, _i, _pd, _i, _u64p, _u64p]
    lib.bef_host_rne53_add.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.bef_host_rne53_add.restype = ctypes.c_uint64
    lib.bef_host_run_pair.argtypes = [_vp, _i, _i, _u64p]
    lib.bef_host_fast_units.argtypes = [_vp, _i, _i, _pd, _i, _u64p]
    lib.bef_host_fast_noise.argtypes = [_vp, _vp, _i, _i, _pd, _i, _u64p]
    lib.bef_host_load_shape.argtypes = [_vp, _vp, _i, _pd, _pd, _i, ctypes.POINTER(ctypes.c_int)]
    return lib


class Emu:
    """The emulation entry points on numpy planes; ``path`` selects a build
    (default: the plain one, built on first use)."""

    def __init__(self, path: str | None = None):
        global _default
        if path is None:
            with _lock:
                if _default is None:
                    d = tempfile.mkdtemp(prefix="bef_emu_")
                    _default = _build.build_host_emu(os.path.join(d, "libbef_emu.so"))
                path = _default
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise ValueError(f"{what} returned {rc}")

    def plane_units(self, plane: np.ndarray, bpc: int, w: int | None = None, dbg: int = 0):
        """[S1, S2_exact, S2_cpu] of the general walk on one plane."""
        h, stride = plane.shape
        w = stride if w is None else w
        out = (ctypes.c_uint64 * 3)()
        self._check(self.lib.bef_host_plane_units(plane.ctypes.data, w, h, stride, bpc, dbg, out),
                    "bef_host_plane_units")
        return list(out)

    def noise_units(self, ref: np.ndarray, dis: np.ndarray, bpc: int, w: int | None = None):
        h, stride = ref.shape
        w = stride if w is None else w
        bits, ex = ctypes.c_uint64(), ctypes.c_uint64()
        self._check(self.lib.bef_host_noise_units(ref.ctypes.data, dis.ctypes.data, w, h, stride,
                                                  bpc, ctypes.byref(bits), ctypes.byref(ex)),
                    "bef_host_noise_units")
        return bits.value, ex.value

    def fast_units(self, plane: np.ndarray, bpc: int, w: int | None = None):
        """[handled, S_cpu, S_exact] of the fast path's decisions on one plane."""
        h, stride = plane.shape
        w = stride if w is None else w
        out = (ctypes.c_uint64 * 3)()
        self._check(self.lib.bef_host_fast_units(plane.ctypes.data, w, h, stride, bpc, out),
                    "bef_host_fast_units")
        return list(out)

    def fast_noise(self, ref: np.ndarray, dis: np.ndarray, bpc: int, w: int | None = None):
        """[handled, bits of the noise double in units, exact] of the fast noise."""
        h, stride = ref.shape
        w = stride if w is None else w
        out = (ctypes.c_uint64 * 3)()
        self._check(self.lib.bef_host_fast_noise(ref.ctypes.data, dis.ctypes.data, w, h, stride,
                                                 bpc, out), "bef_host_fast_noise")
        return list(out)

    def rne53_add(self, s: int, t: int) -> int:
        return int(self.lib.bef_host_rne53_add(s, t))

    def run_pair(self, terms: np.ndarray, e: int):
        t = np.ascontiguousarray(terms, dtype=np.uint32)
        out = (ctypes.c_uint64 * 2)()
        self._check(self.lib.bef_host_run_pair(t.ctypes.data, t.size, e, out), "bef_host_run_pair")
        return list(out)

    def load_shape(self, ref_addr: int, dis_addr: int, w: int, stride: int, frame_pitch: int,
                   nframes: int):
        """(bytes per load, load slots per group) the row kernel uses for
        planes at these addresses (alignment only; nothing is read)."""
        out = (ctypes.c_int * 2)()
        self._check(self.lib.bef_host_load_shape(ctypes.c_void_p(ref_addr),
                                                 ctypes.c_void_p(dis_addr), w, stride,
                                                 frame_pitch, nframes, out),
                    "bef_host_load_shape")
        return out[0], out[1]
