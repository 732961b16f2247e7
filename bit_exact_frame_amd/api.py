"""Thin ctypes binding of libbef.so (include/bef.h), same names as the C ABI.

Argument marshalling only: tensors in, pointers and sizes to the C entry
points, results out.  Every step of the reductions runs in the library's
HIP kernels.  If libbef.so is missing this module raises at import: there is
no CPU fallback.

Planes are torch tensors in device memory (uint8 for bpc 8, uint16
otherwise), shaped (h, stride) for one frame or (F, h, stride) for a batch,
C-contiguous; ``w`` defaults to the last dimension.
"""
from __future__ import annotations

import atexit
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbef.so")

# torch first: its HIP runtime (libamdhip64.so.7, same soname as the system
# one) must be the one libbef.so binds to, so that a single runtime owns the
# device in the process.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise RuntimeError(
        f"{LIB_PATH} is missing: build it first "
        "(python -m bit_exact_frame_amd.build or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _pd, _u = ctypes.c_void_p, ctypes.c_int, ctypes.c_ssize_t, ctypes.c_uint
_dp = ctypes.POINTER(ctypes.c_double)
_u64p = ctypes.POINTER(ctypes.c_uint64)

_lib.moment_frame.argtypes = [_vp, _vp, _i, _i, _pd, _i, _dp]
_lib.psnr_noise.argtypes = [_vp, _vp, _i, _i, _pd, _i, _dp]
_lib.bef_frames.argtypes = [_vp, _vp, _i, _i, _pd, _pd, _i, _i, _vp, _dp, _dp]
_lib.bef_frames_async.argtypes = [_vp, _vp, _i, _i, _pd, _pd, _i, _i, _vp, _vp]
_lib.bef_frames_noalloc.argtypes = [_vp, _vp, _i, _i, _pd, _pd, _i, _i, _vp, _vp]
_lib.bef_frames_units.argtypes = [_vp, _vp, _i, _i, _pd, _pd, _i, _i, _vp, _u64p]
_lib.bef_read_ceiling.argtypes = [_vp, _vp, _i, _i, _pd, _pd, _i, _vp, _vp]
_lib.bef_frames_host.argtypes = [_vp, _vp, _i, _i, _pd, _pd, _i, _i, _i, _dp, _dp]
_lib.bef_planes.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _dp]
_lib.bef_pipe_submit.argtypes = [_vp, _vp, _i, _i, _pd, _pd, _i, _i, _vp, _vp]
_lib.bef_pipe_join.argtypes = [_i, _vp]
_lib.bef_pipe_set_walk_cus.argtypes = [_i]
for _n in ("moment_frame", "psnr_noise", "bef_frames", "bef_frames_async", "bef_frames_noalloc",
           "bef_frames_units", "bef_read_ceiling", "bef_frames_host", "bef_planes",
           "bef_pipe_submit", "bef_pipe_join", "bef_pipe_set_walk_cus"):
    getattr(_lib, _n).restype = _i
_lib.bef_last_error.restype = ctypes.c_char_p
_lib.bef_walk_paths.argtypes = [_vp, _i]
_lib.bef_walk_paths.restype = _i
_lib.bef_debug_set.argtypes = [_u]
_lib.bef_debug_set.restype = _u
_lib.bef_timing_enable.argtypes = [_i]
_lib.bef_timing_read.argtypes = [_i, _dp, ctypes.POINTER(ctypes.c_long)]
_lib.bef_release.restype = None

# The library's streams, events and device memory go before the HIP runtime
# is torn down at exit.
atexit.register(_lib.bef_release)
_lib.bef_timing_reset.restype = None

DBG_PLAN_WRONG = 1
DBG_PLAN_NONE = 2
DBG_TERMS_ONLY = 4
DBG_FORCE_ROUND = 8
DBG_NO_STRETCH = 16
DBG_NO_CLOSED_FORM = 32
DBG_SPLIT_LAUNCH = 64

KERNELS = {"rows": 0, "plan": 1, "pairs": 2, "walk": 3, "ceiling": 4}


class BefError(RuntimeError):
    pass


def lib():
    return _lib


def last_error() -> str:
    return _lib.bef_last_error().decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise BefError(f"{what} returned {rc}: {last_error()}")


def _geom(t, bpc, w):
    import torch
    if not t.is_cuda:
        raise BefError("planes must be device tensors")
    want = torch.uint8 if bpc == 8 else torch.uint16
    if t.dtype != want:
        raise BefError(f"bpc {bpc} needs {want} planes, got {t.dtype}")
    if not t.is_contiguous():
        raise BefError("planes must be contiguous")
    h, stride = t.shape[-2], t.shape[-1]
    f = t.shape[0] if t.dim() == 3 else 1
    return f, h, stride, (stride if w is None else int(w))


def _pair(ref, dis, bpc, w):
    """Geometry of a (ref, dis) pair of device planes: both must pass the
    same checks and have the same shape on the same device (the library
    reads dis with ref's geometry)."""
    geom = _geom(ref, bpc, w)
    _geom(dis, bpc, w)
    if tuple(dis.shape) != tuple(ref.shape):
        raise BefError(f"ref and dis shapes differ: {tuple(ref.shape)} and {tuple(dis.shape)}")
    if dis.device != ref.device:
        raise BefError(f"ref on {ref.device}, dis on {dis.device}")
    if not 1 <= geom[3] <= geom[2]:
        raise BefError(f"w={geom[3]} outside 1..{geom[2]} (the planes' last dimension)")
    return geom


def _stream_ptr(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def moment_frame(ref, dis, bpc: int, w: int | None = None):
    """Four moments of one frame: [ref_1st, dis_1st, ref_2nd, dis_2nd]."""
    _, h, stride, w = _pair(ref, dis, bpc, w)
    out = (ctypes.c_double * 4)()
    _check(_lib.moment_frame(ref.data_ptr(), dis.data_ptr(), w, h, stride, bpc, out),
           "moment_frame")
    return list(out)


def psnr_noise(ref, dis, bpc: int, w: int | None = None):
    """[noise, mse] of one frame."""
    _, h, stride, w = _pair(ref, dis, bpc, w)
    out = (ctypes.c_double * 2)()
    _check(_lib.psnr_noise(ref.data_ptr(), dis.data_ptr(), w, h, stride, bpc, out),
           "psnr_noise")
    return list(out)


def bef_frames(ref, dis, bpc: int, w: int | None = None, stream=None):
    """Batch: returns (moments float64[F,4], psnr float64[F,2])."""
    f, h, stride, w = _pair(ref, dis, bpc, w)
    mom = np.zeros((f, 4), np.float64)
    ps = np.zeros((f, 2), np.float64)
    _check(_lib.bef_frames(ref.data_ptr(), dis.data_ptr(), w, h, stride, h * stride, f,
                           bpc, _stream_ptr(stream), mom.ctypes.data_as(_dp),
                           ps.ctypes.data_as(_dp)), "bef_frames")
    return mom, ps


def bef_planes(refs, diss, bpc: int, ws=None, stream=None):
    """Several planes of each frame (e.g. Y, Cb, Cr), one call: refs[p] and
    diss[p] are device tensors (F, h_p, stride_p) (or (h_p, stride_p)), with
    the same F for every plane; ws[p] the width (default stride_p).
    Returns float64 [P, F, 7]: ref_1st, dis_1st, ref_2nd, dis_2nd, noise,
    mse, psnr_db (the dB value is a reading: parity unpinned)."""
    n = len(refs)
    if n != len(diss) or not 1 <= n <= 4:
        raise BefError("refs and diss must list the same 1..4 planes")
    ws = [None] * n if ws is None else list(ws)
    geo = [_pair(refs[p], diss[p], bpc, ws[p]) for p in range(n)]
    f = geo[0][0]
    if any(g[0] != f for g in geo):
        raise BefError("every plane needs the same number of frames")
    P = ctypes.c_void_p * n
    rp = P(*[refs[p].data_ptr() for p in range(n)])
    dp = P(*[diss[p].data_ptr() for p in range(n)])
    w = (ctypes.c_int * n)(*[g[3] for g in geo])
    h = (ctypes.c_int * n)(*[g[1] for g in geo])
    st = (ctypes.c_ssize_t * n)(*[g[2] for g in geo])
    pt = (ctypes.c_ssize_t * n)(*[g[1] * g[2] for g in geo])
    out = np.zeros((n, f, 7), np.float64)
    _check(_lib.bef_planes(rp, dp, w, h, st, pt, n, f, bpc, _stream_ptr(stream),
                           out.ctypes.data_as(_dp)), "bef_planes")
    return out


def _host_geom(t, bpc, w):
    want = np.uint8 if bpc == 8 else np.uint16
    if isinstance(t, np.ndarray):
        if t.dtype != want or not t.flags.c_contiguous:
            raise BefError(f"bpc {bpc} needs C-contiguous {want.__name__} host planes")
        ptr = t.ctypes.data
    else:  # a CPU torch tensor (pinned or not)
        import torch
        if t.is_cuda or not t.is_contiguous():
            raise BefError("host planes must be contiguous CPU tensors or arrays")
        if t.dtype != (torch.uint8 if bpc == 8 else torch.uint16):
            raise BefError(f"bpc {bpc} needs {want.__name__} host planes")
        ptr = t.data_ptr()
    h, stride = t.shape[-2], t.shape[-1]
    f = t.shape[0] if t.ndim == 3 else 1
    return ptr, f, h, stride, (stride if w is None else int(w))


def bef_frames_host(ref, dis, bpc: int, w: int | None = None, device: int = 0):
    """Batch from HOST planes (numpy arrays or CPU tensors, (F, h, stride) or
    (h, stride)): returns (moments float64[F,4], psnr float64[F,2])."""
    pr, f, h, stride, w = _host_geom(ref, bpc, w)
    pd, f2, h2, stride2, _ = _host_geom(dis, bpc, w)
    if (f2, h2, stride2) != (f, h, stride):
        raise BefError("ref and dis shapes differ")
    mom = np.zeros((f, 4), np.float64)
    ps = np.zeros((f, 2), np.float64)
    _check(_lib.bef_frames_host(ctypes.c_void_p(pr), ctypes.c_void_p(pd), w, h, stride,
                                h * stride, f, bpc, int(device), mom.ctypes.data_as(_dp),
                                ps.ctypes.data_as(_dp)), "bef_frames_host")
    return mom, ps


def bef_frames_async(ref, dis, bpc: int, out, w: int | None = None, stream=None):
    """Batch into the float64 device tensor ``out`` [F,6]; no sync."""
    import torch
    f, h, stride, w = _pair(ref, dis, bpc, w)
    if out.dtype != torch.float64 or not out.is_cuda or out.numel() < 6 * f:
        raise BefError("out must be a float64 device tensor of at least 6*F")
    _check(_lib.bef_frames_async(ref.data_ptr(), dis.data_ptr(), w, h, stride, h * stride,
                                 f, bpc, _stream_ptr(stream), ctypes.c_void_p(out.data_ptr())),
           "bef_frames_async")


def bef_frames_noalloc(ref, dis, bpc: int, out, w: int | None = None, stream=None):
    """As bef_frames_async, with the library's static scratch: the call
    allocates nothing.  ``out``: float64 device tensor [F,6]."""
    import torch
    f, h, stride, w = _pair(ref, dis, bpc, w)
    if out.dtype != torch.float64 or not out.is_cuda or out.numel() < 6 * f:
        raise BefError("out must be a float64 device tensor of at least 6*F")
    _check(_lib.bef_frames_noalloc(ref.data_ptr(), dis.data_ptr(), w, h, stride, h * stride,
                                   f, bpc, _stream_ptr(stream), ctypes.c_void_p(out.data_ptr())),
           "bef_frames_noalloc")


def bef_pipe_submit(ref, dis, bpc: int, out, w: int | None = None, stream=None):
    """Pipelined batch into the float64 device tensor ``out`` [F,6]: complete
    once ``stream`` has passed a later bef_pipe_join."""
    import torch
    f, h, stride, w = _pair(ref, dis, bpc, w)
    if out.dtype != torch.float64 or not out.is_cuda or out.numel() < 6 * f:
        raise BefError("out must be a float64 device tensor of at least 6*F")
    _check(_lib.bef_pipe_submit(ref.data_ptr(), dis.data_ptr(), w, h, stride, h * stride,
                                f, bpc, _stream_ptr(stream), ctypes.c_void_p(out.data_ptr())),
           "bef_pipe_submit")


def bef_pipe_join(device: int = 0, stream=None):
    """Makes ``stream`` wait for every pipelined batch of ``device``."""
    _check(_lib.bef_pipe_join(int(device), _stream_ptr(stream)), "bef_pipe_join")


def bef_pipe_set_walk_cus(n: int) -> int:
    """Sets the walk stream's CUs (0: unchanged); returns the previous count."""
    rc = _lib.bef_pipe_set_walk_cus(int(n))
    if rc < 0:
        raise BefError(f"bef_pipe_set_walk_cus returned {rc}: {last_error()}")
    return rc


def bef_pipe_walk_cus() -> int:
    return bef_pipe_set_walk_cus(0)


def bef_frames_units(ref, dis, bpc: int, w: int | None = None, stream=None):
    """Batch diagnostics: uint64[F,8] integer sums in units."""
    f, h, stride, w = _pair(ref, dis, bpc, w)
    units = np.zeros((f, 8), np.uint64)
    _check(_lib.bef_frames_units(ref.data_ptr(), dis.data_ptr(), w, h, stride, h * stride,
                                 f, bpc, _stream_ptr(stream), units.ctypes.data_as(_u64p)),
           "bef_frames_units")
    return units


def bef_read_ceiling(ref, dis, out, w: int | None = None, stream=None):
    """Diagnostic read-only pass over 16-bit planes (the row pass's memory
    side); ``out`` is a uint32 device tensor of at least F*h words."""
    import torch
    f, h, stride, w = _pair(ref, dis, 16, w)
    if out.dtype != torch.int32 and out.dtype != torch.uint32:
        raise BefError("out must be a 32-bit integer device tensor")
    if not out.is_cuda or out.numel() < f * h:
        raise BefError("out must be a device tensor of at least F*h words")
    _check(_lib.bef_read_ceiling(ref.data_ptr(), dis.data_ptr(), w, h, stride, h * stride, f,
                                 _stream_ptr(stream), ctypes.c_void_p(out.data_ptr())),
           "bef_read_ceiling")


PATHS = {0: "sums", 1: "fast", 2: "general", 3: "chain", 4: "skipped"}


def bef_walk_paths():
    """Walk path of each (frame, job) of the last synchronous batch, as a
    uint8 array [F, 3] (jobs: ref moments, dis moments, noise; codes in
    PATHS)."""
    n = _lib.bef_walk_paths(None, 0)
    out = np.zeros(n, np.uint8)
    if n:
        _lib.bef_walk_paths(ctypes.c_void_p(out.ctypes.data), n)
    return out.reshape(-1, 3)


def bef_debug_set(flags: int) -> int:
    return int(_lib.bef_debug_set(int(flags)))


def bef_timing_enable(on: bool):
    _lib.bef_timing_enable(1 if on else 0)


def bef_timing_reset():
    _lib.bef_timing_reset()


def bef_timing_read(kernel: str):
    ms = ctypes.c_double()
    n = ctypes.c_long()
    _check(_lib.bef_timing_read(KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)),
           "bef_timing_read")
    return ms.value, n.value


def bef_release():
    _lib.bef_release()
