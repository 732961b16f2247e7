"""The entry point that allocates nothing (needs an MI355X).

bef_frames_noalloc runs the same kernels as bef_frames_async with the
library's static scratch (a fixed device array) instead of its arena.  Its
results must equal bef_frames_async's bit for bit on the same frames, call
after call, also when a call follows a larger one (the array keeps the last
call's contents and no call may depend on them).
"""
from __future__ import annotations

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


def both(api, ref, dis, bpc, w=None):
    """[F,6] results of bef_frames_noalloc and of bef_frames_async."""
    import torch
    f = ref.shape[0]
    r, d = dev(ref), dev(dis)
    a = torch.full((f, 6), -1.0, dtype=torch.float64, device="cuda")
    b = torch.full((f, 6), -2.0, dtype=torch.float64, device="cuda")
    api.bef_frames_noalloc(r, d, bpc, a, w=w)
    torch.cuda.synchronize()
    api.bef_frames_async(r, d, bpc, b, w=w)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_matches_async_larger_then_smaller(api):
    """Calls in a row, each against bef_frames_async: 16 frames of 16-bit
    3840x2160 noise (past 2^53), then 3 of the 10-bit 1920x1080 workload
    (smaller), then 2 of 16-bit 7680x4320 noise (past 2^55: plan and row
    pairs in the scratch), then 2 of 16-bit 4096x2560 near-maximum content
    (in the binade of 2^55: the fast walk's seven-edge form reads the row
    pairs from the scratch), then 1 frame of 8-bit 176x144 (smaller again).
    The 8-bit frame is also checked against the oracle."""
    cases = [(4, 16), (2, 3), (6, 2), (7, 2), (1, 1)]
    for key, nf in cases:
        wl = synth.WORKLOADS[key]
        ref, dis = synth.make_frames(key, frames=nf)
        say(f"[gpu] noalloc {wl.name} frames={nf}")
        a, b = both(api, ref, dis, wl.bpc, w=wl.w)
        assert (bits(a) == bits(b)).all(), (wl.name, a, b)
        if key == 1:
            emom, eps = oracle.Oracle().frames(ref, dis, wl.bpc, w=wl.w)
            assert (bits(a[:, :4]) == bits(emom)).all() and (bits(a[:, 4:]) == bits(eps)).all()


def test_noalloc_padded_and_debug_paths(api):
    """A padded 12-bit batch, then wrong plans forced on 4K half-range
    frames (general walk, row pairs from lane runs), against the async
    call under the same setting."""
    ref, dis = synth.make_frames(3, frames=4)
    say("[gpu] noalloc 12-bit padded frames=4")
    a, b = both(api, ref, dis, 12, w=2560)
    assert (bits(a) == bits(b)).all()
    ref, dis = synth.make_frames(5, frames=2)
    old = api.bef_debug_set(api.DBG_PLAN_WRONG | api.DBG_NO_CLOSED_FORM)
    try:
        say("[gpu] noalloc half-range frames=2, wrong plans, no closed forms")
        a, b = both(api, ref, dis, 16)
    finally:
        api.bef_debug_set(old)
    assert (bits(a) == bits(b)).all()


def test_noalloc_rejects_a_batch_beyond_the_static_scratch(api):
    """A batch whose scratch would pass the fixed array is refused before
    any launch, with the sizes in the message; a batch that fits runs."""
    import torch
    h, w = 2160, 8
    big = np.zeros((200, h, w), dtype=np.uint16)
    r, d = dev(big), dev(big)
    out = torch.zeros((200, 6), dtype=torch.float64, device="cuda")
    with pytest.raises(api.BefError, match="static scratch"):
        api.bef_frames_noalloc(r, d, 16, out)
    say("[gpu] noalloc 100 frames of 2160 rows")
    a, b = both(api, big[:100], big[:100], 16)
    assert (bits(a) == bits(b)).all() and (a == 0.0).all()
