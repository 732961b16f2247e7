"""The Python binding refuses a mismatched distorted plane before any C call
(CPU only).

The library reads dis with ref's geometry, so every device entry point's
binding checks dis as it checks ref (device tensor, dtype of the bit depth,
contiguous) and that both have one shape on one device.  Stand-in tensors
report a device; any attempt to pass their address on fails the test.
"""
from __future__ import annotations

import pytest
import torch


class DevPlane:
    """A CPU tensor that presents itself as a device plane; data_ptr() must
    never be reached."""

    def __init__(self, t, device="cuda:0", cuda=True):
        self.t = t
        self.is_cuda = cuda
        self.device = torch.device(device)
        self.dtype = t.dtype
        self.shape = t.shape

    def dim(self):
        return self.t.dim()

    def is_contiguous(self):
        return self.t.is_contiguous()

    def data_ptr(self):
        raise AssertionError("a C call was reached with mismatched planes")


@pytest.fixture(scope="module")
def api():
    from bit_exact_frame_amd import api as _api
    return _api


def calls(api):
    out = DevPlane(torch.zeros((3, 6), dtype=torch.float64))
    ceil_out = DevPlane(torch.zeros(3 * 8, dtype=torch.int32))
    return {
        "moment_frame": lambda r, d, b: api.moment_frame(r, d, b),
        "psnr_noise": lambda r, d, b: api.psnr_noise(r, d, b),
        "bef_frames": lambda r, d, b: api.bef_frames(r, d, b),
        "bef_frames_units": lambda r, d, b: api.bef_frames_units(r, d, b),
        "bef_frames_async": lambda r, d, b: api.bef_frames_async(r, d, b, out),
        "bef_frames_noalloc": lambda r, d, b: api.bef_frames_noalloc(r, d, b, out),
        "bef_pipe_submit": lambda r, d, b: api.bef_pipe_submit(r, d, b, out),
        "bef_read_ceiling": lambda r, d, b: api.bef_read_ceiling(r, d, ceil_out),
    }


def bad_dis():
    """(label, dis) pairs that must be refused next to a (3, 8, 16) uint16 ref."""
    u16 = torch.zeros((3, 8, 16), dtype=torch.uint16)
    return [
        ("fewer frames", DevPlane(u16[:2])),
        ("fewer rows", DevPlane(torch.zeros((3, 7, 16), dtype=torch.uint16))),
        ("narrower rows", DevPlane(torch.zeros((3, 8, 15), dtype=torch.uint16))),
        ("uint8 samples", DevPlane(torch.zeros((3, 8, 16), dtype=torch.uint8))),
        ("not contiguous", DevPlane(torch.zeros((3, 16, 8), dtype=torch.uint16).transpose(1, 2))),
        ("host memory", DevPlane(u16, device="cpu", cuda=False)),
        ("another device", DevPlane(u16, device="cuda:1")),
    ]


@pytest.mark.parametrize("entry", ["moment_frame", "psnr_noise", "bef_frames", "bef_frames_units",
                                   "bef_frames_async", "bef_frames_noalloc", "bef_pipe_submit",
                                   "bef_read_ceiling"])
def test_mismatched_dis_is_refused(api, entry):
    ref = DevPlane(torch.zeros((3, 8, 16), dtype=torch.uint16))
    fn = calls(api)[entry]
    for label, dis in bad_dis():
        with pytest.raises(api.BefError):
            fn(ref, dis, 16)
        # the same mistake on the ref side is refused too
        if label not in ("fewer frames", "fewer rows", "narrower rows"):
            with pytest.raises(api.BefError):
                fn(dis, ref, 16)


def test_width_beyond_the_planes_is_refused(api):
    ref = DevPlane(torch.zeros((2, 4, 16), dtype=torch.uint16))
    dis = DevPlane(torch.zeros((2, 4, 16), dtype=torch.uint16))
    with pytest.raises(api.BefError, match="outside"):
        api.bef_frames(ref, dis, 16, w=17)
    with pytest.raises(api.BefError, match="outside"):
        api.bef_frames(ref, dis, 16, w=0)


def test_planes_binding_checks(api):
    """bef_planes refuses planes with different frame counts, more than four
    planes, and a mismatched dis in any plane, before any C call."""
    y = DevPlane(torch.zeros((2, 8, 16), dtype=torch.uint16))
    c = DevPlane(torch.zeros((2, 4, 8), dtype=torch.uint16))
    c1 = DevPlane(torch.zeros((1, 4, 8), dtype=torch.uint16))
    with pytest.raises(api.BefError, match="frames"):
        api.bef_planes([y, c1], [y, c1], 16)
    with pytest.raises(api.BefError):
        api.bef_planes([y, c, c, c, c], [y, c, c, c, c], 16)
    with pytest.raises(api.BefError):
        api.bef_planes([y, c], [y, DevPlane(torch.zeros((2, 4, 7), dtype=torch.uint16))], 16)
    with pytest.raises(api.BefError):
        api.bef_planes([y, c], [y], 16)

