"""Several planes per frame through one call (needs an MI355X).

bef_planes takes the luma and chroma planes of 4:2:0 pictures (odd luma
sizes, so the chroma planes are ceil(w/2) x ceil(h/2)), each with its own
geometry and padding, and returns per plane the float_moment and float_psnr
results of every frame and a PSNR in dB.  The moments, noise and MSE of every
plane must be the oracle's bits (each plane is reduced as the CPU reduces a
luma plane: ADR-1497, Context; ADR-1499, Context).  The dB value is a
reading of the pages, which give no formula (parity unpinned): it must
match the oracle's reading within the rounding bound of the log.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle
from bit_exact_frame_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_exact_frame_amd import api as _api
    _api.bef_debug_set(0)
    return _api


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(x):
    return np.asarray(x, dtype=np.float64).view(np.uint64)


CASES = [
    # (label, bpc, luma w, h, pad, frames, lo, hi, dis noise)
    ("8-bit 177x145", 8, 177, 145, 3, 4, 0, None, None),
    ("10-bit 1921x1081 noise 8", 10, 1921, 1081, 7, 3, 0, None, 8.0),
    ("16-bit 3841x2161 full range", 16, 3841, 2161, 0, 2, 0, None, None),
    ("16-bit 3841x2161 half range", 16, 3841, 2161, 5, 2, 32768, None, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_yuv420_planes_match_the_oracle(api, case):
    label, bpc, w, h, pad, nf, lo, hi, noise = case
    planes = synth.yuv420_frames(w * 7 + h, nf, w, h, bpc, pad=pad, lo=lo, hi=hi, noise=noise)
    if label.startswith("8-bit"):
        planes[2] = (planes[2][0], planes[2][0].copy())  # Cr: dis == ref, MSE 0
    widths = [w, (w + 1) // 2, (w + 1) // 2]
    say(f"[gpu] planes {label}")
    got = api.bef_planes([dev(r) for r, _ in planes], [dev(d) for _, d in planes], bpc, ws=widths)
    assert got.shape == (3, nf, 7)
    orc = oracle.Oracle()
    for p, (r, d) in enumerate(planes):
        emom, eps = orc.frames(r, d, bpc, w=widths[p])
        assert (bits(got[p, :, :4]) == bits(emom)).all(), (label, p, got[p, :, :4], emom)
        assert (bits(got[p, :, 4:6]) == bits(eps)).all(), (label, p, got[p, :, 4:6], eps)
        for f in range(nf):
            want = orc.psnr_db(eps[f, 1], bpc)
            db = got[p, f, 6]
            if math.isinf(want):
                assert db == want, (label, p, f, db)
            else:
                assert abs(db - want) <= 4 * math.ulp(want) + 1e-15, (label, p, f, db, want)
    # the luma plane alone through the batch call gives the same bits
    mom, ps = api.bef_frames(dev(planes[0][0]), dev(planes[0][1]), bpc, w=w)
    assert (bits(mom) == bits(got[0, :, :4])).all() and (bits(ps) == bits(got[0, :, 4:6])).all()


def test_planes_past_2_55_and_bad_arguments(api):
    """One 8K plane past 2^55 with a small second plane (row pairs, general
    walk) against the batch call; mismatched frame counts are refused."""
    r8, d8 = synth.make_frames(6, frames=1)
    rs, ds = synth.uniform_planes(55, 1, 33, 70, 75, 16)
    say("[gpu] planes 8K + 70x33")
    got = api.bef_planes([dev(r8), dev(rs)], [dev(d8), dev(ds)], 16, ws=[7680, 70])
    for p, (r, d, w) in enumerate(((r8, d8, 7680), (rs, ds, 70))):
        mom, ps = api.bef_frames(dev(r), dev(d), 16, w=w)
        assert (bits(mom) == bits(got[p, :, :4])).all() and (bits(ps) == bits(got[p, :, 4:6])).all()
    r2, d2 = synth.uniform_planes(56, 2, 33, 70, 70, 16)
    with pytest.raises(api.BefError):
        api.bef_planes([dev(r8), dev(r2)], [dev(d8), dev(d2)], 16, ws=[7680, 70])
