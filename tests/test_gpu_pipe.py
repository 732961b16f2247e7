"""Pipelined batches vs the oracle and the one-stream path (needs an MI355X).

bef_pipe_submit runs the same kernels as bef_frames_async, spread over the
library's own streams: two row streams that take turns, a walk stream on
CUs of its own, four scratch slots reused in turn.  Every batch must still
return the CPU loop's bits (ADR-1497, Consequences; ADR-1499, Consequences:
tolerance 0), whatever the order in which its neighbours' kernels ran:
more batches than slots, both row streams, slots that grow while earlier
batches are in flight, batches that need the plan and the row pairs, a
change of the walk's CUs between batches, and the legacy NULL stream.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

import boundary
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
    yield _api
    _api.bef_debug_set(0)
    _api.bef_pipe_set_walk_cus(16)


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(x):
    return np.asarray(x, dtype=np.float64).view(np.uint64)


def out_for(f):
    import torch
    return torch.full((f, 6), -1.0, dtype=torch.float64, device="cuda")


def run(api, batches, stream=None):
    """Submit every (ref, dis, bpc, w, out) on ``stream``, join, wait."""
    import torch
    for ref, dis, bpc, w, out in batches:
        api.bef_pipe_submit(ref, dis, bpc, out, w=w, stream=stream)
    api.bef_pipe_join(0, stream)
    torch.cuda.synchronize()


def same_as(api, got, ref, dis, bpc, w, label):
    """``got`` [F,6] against bef_frames on the same device planes."""
    mom, ps = api.bef_frames(ref, dis, bpc, w=w)
    g = got.cpu().numpy()
    assert (bits(g[:, :4]) == bits(mom)).all() and (bits(g[:, 4:]) == bits(ps)).all(), (
        label, g, mom, ps)


def boundary_pair(kind):
    p = boundary.build(kind)
    ref = p[None]
    dis = np.ascontiguousarray(np.flip(p, axis=1))[None]
    return ref, dis


def test_pipe_mixed_batches_match_oracle(api, orc):
    """Eleven batches of six shapes (more than the four slots, both row
    streams), each into its own output, against the oracle: 8-bit 176x144,
    10-bit 1920x1080, padded 12-bit 2560x1440, 16-bit half range and four
    boundary frames (exact sums 2^53 - 1, 2^53, 2^53 then three ties, 2^54
    + 7)."""
    import torch
    cases = []
    for key, nf in ((1, 4), (2, 3), (3, 2), (5, 2)):
        wl = synth.WORKLOADS[key]
        ref, dis = synth.make_frames(key, frames=nf)
        cases.append((wl.name, ref, dis, wl.bpc, wl.w))
    for kind in ("b53m1", "b53", "b53p3", "b54p7"):
        ref, dis = boundary_pair(kind)
        cases.append((kind, ref, dis, 16, None))
    order = [0, 4, 1, 5, 2, 6, 3, 7, 0, 5, 2]
    st = torch.cuda.Stream()
    batches, want = [], []
    for k in order:
        name, ref, dis, bpc, w = cases[k]
        batches.append((dev(ref), dev(dis), bpc, w, out_for(ref.shape[0])))
        want.append((name, ref, dis, bpc, w))
    torch.cuda.synchronize()
    say(f"[gpu] pipe mixed: {len(batches)} batches {[cases[k][0] for k in order]}")
    run(api, batches, st)
    for (name, ref, dis, bpc, w), b in zip(want, batches):
        emom, eps = orc.frames(ref, dis, bpc, w=w)
        g = b[4].cpu().numpy()
        assert (bits(g[:, :4]) == bits(emom)).all(), (name, g[:, :4], emom)
        assert (bits(g[:, 4:]) == bits(eps)).all(), (name, g[:, 4:], eps)


def test_pipe_slot_growth_and_shared_output(api):
    """Small, large, small batches in a row, so that a slot grows while
    earlier batches are in flight (the library first waits for them); nine
    batches of full-range 4K noise (16 frames, past 2^53) share one output,
    whose last batch decides it.  Against bef_frames on the same planes."""
    import torch
    w1 = synth.WORKLOADS[1]
    s_ref, s_dis = synth.make_frames(1)
    w4 = synth.WORKLOADS[4]
    l_ref, l_dis = synth.make_frames(4)
    sr, sd = dev(s_ref), dev(s_dis)
    lr, ld = dev(l_ref), dev(l_dis)
    # a second large batch: frames in another order
    lr2, ld2 = dev(l_ref[::-1]), dev(l_dis[::-1])
    small = [out_for(4) for _ in range(3)]
    shared = out_for(16)
    st = torch.cuda.Stream()
    api.bef_pipe_set_walk_cus(16)
    torch.cuda.synchronize()
    batches = [(sr, sd, 8, w1.w, small[0])]
    for k in range(9):
        batches.append((lr2, ld2, 16, w4.w, shared) if k < 8 else (lr, ld, 16, w4.w, shared))
        if k == 4:
            batches.append((sr, sd, 8, w1.w, small[1]))
    batches.append((sr, sd, 8, w1.w, small[2]))
    say(f"[gpu] pipe growth: {len(batches)} batches, 8-bit 176x144 and 16-bit 3840x2160 x16")
    run(api, batches, st)
    same_as(api, shared, lr, ld, 16, w4.w, "shared output, last batch")
    for k, o in enumerate(small):
        same_as(api, o, sr, sd, 8, w1.w, f"small batch {k}")


def test_pipe_past_2_55_and_forced_plans(api):
    """Batches that need the plan and the row pairs: 16-bit 7680x4320 noise
    (past 2^55) and 4096x2560 near-maximum frames, then 4K half-range frames
    with wrong plans forced (general walk, lane runs)."""
    import torch
    st = torch.cuda.Stream()
    planes = []
    for key, nf in ((6, 2), (7, 2)):
        wl = synth.WORKLOADS[key]
        ref, dis = synth.make_frames(key, frames=nf)
        planes.append((wl.name, dev(ref), dev(dis), wl.bpc, wl.w))
    torch.cuda.synchronize()
    outs = [out_for(p[1].shape[0]) for p in planes]
    say("[gpu] pipe past 2^55: " + ", ".join(p[0] for p in planes) + " x2 each")
    run(api, [(r, d, b, w, o) for (_, r, d, b, w), o in zip(planes + planes, outs + outs)], st)
    for (name, r, d, b, w), o in zip(planes, outs):
        same_as(api, o, r, d, b, w, name)
    wl = synth.WORKLOADS[5]
    ref, dis = synth.make_frames(5, frames=3)
    r, d = dev(ref), dev(dis)
    want = out_for(3)
    api.bef_frames_async(r, d, 16, want, w=wl.w)
    torch.cuda.synchronize()
    old = api.bef_debug_set(api.DBG_PLAN_WRONG)
    try:
        o1, o2 = out_for(3), out_for(3)
        say("[gpu] pipe half range with wrong plans")
        run(api, [(r, d, 16, wl.w, o1), (r, d, 16, wl.w, o2)], st)
    finally:
        api.bef_debug_set(old)
    assert (bits(o1.cpu().numpy()) == bits(want.cpu().numpy())).all()
    assert (bits(o2.cpu().numpy()) == bits(want.cpu().numpy())).all()


def test_pipe_walk_cus_change_and_null_stream(api, orc):
    """The walk's CUs changed between batches (the library waits for the
    batches in flight and rebuilds its streams), then batches submitted and
    joined on the legacy NULL stream; the 8-bit workload against the
    oracle."""
    import torch
    wl = synth.WORKLOADS[1]
    ref, dis = synth.make_frames(1)
    emom, eps = orc.frames(ref, dis, 8, w=wl.w)
    r, d = dev(ref), dev(dis)
    st = torch.cuda.Stream()
    outs = [out_for(4) for _ in range(4)]
    for k, cus in enumerate((8, 24)):
        api.bef_pipe_set_walk_cus(cus)
        say(f"[gpu] pipe walk CUs {cus}")
        api.bef_pipe_submit(r, d, 8, outs[k], stream=st)
    api.bef_pipe_join(0, st)
    st.synchronize()
    say("[gpu] pipe on the NULL stream")
    api.bef_pipe_submit(r, d, 8, outs[2], stream=0)
    api.bef_pipe_submit(r, d, 8, outs[3], stream=0)
    api.bef_pipe_join(0, 0)
    torch.cuda.synchronize()
    api.bef_pipe_set_walk_cus(16)
    for o in outs:
        g = o.cpu().numpy()
        assert (bits(g[:, :4]) == bits(emom)).all() and (bits(g[:, 4:]) == bits(eps)).all()


def test_pipe_bad_arguments(api):
    """Errors come back as codes with a message; nothing is enqueued."""
    import torch
    lib = api.lib()
    wl = synth.WORKLOADS[1]
    ref, dis = synth.make_frames(1, frames=1)
    r, d = dev(ref), dev(dis)
    rc = lib.bef_pipe_submit(r.data_ptr(), d.data_ptr(), wl.w, wl.h, wl.stride,
                             wl.h * wl.stride, 1, 8, None, None)
    assert rc < 0 and "dev_results" in api.last_error()
    out = out_for(1)
    rc = lib.bef_pipe_submit(r.data_ptr(), d.data_ptr(), wl.w, wl.h, wl.stride - 1,
                             wl.h * wl.stride, 1, 8, None, ctypes.c_void_p(out.data_ptr()))
    assert rc < 0 and "stride" in api.last_error()
    with pytest.raises(api.BefError):
        api.bef_pipe_set_walk_cus(-1)
    with pytest.raises(api.BefError):
        api.bef_pipe_set_walk_cus(129)
    assert api.bef_pipe_walk_cus() == 16
    with pytest.raises(api.BefError):
        api.bef_pipe_join(-1)
    torch.cuda.synchronize()


def test_pipe_random_batches_match_oracle(api, orc):
    """Forty seeded batches of random geometry submitted back to back (1-5
    frames, widths 1-2500 with padded strides, 1-300 rows, every bit depth
    from 8 to 16, uniform or near-maximum content), so that slots, row
    streams and slot growth interleave in many orders; each against the
    oracle."""
    import torch
    rng = np.random.default_rng(20261202)
    st = torch.cuda.Stream()
    batches, want = [], []
    for n in range(40):
        bpc = int(rng.integers(8, 17))
        f = int(rng.integers(1, 6))
        w = int(rng.integers(1, 2501))
        h = int(rng.integers(1, 301))
        stride = w + int(rng.integers(0, 40))
        top = (1 << bpc) - 1
        dt = np.uint8 if bpc == 8 else np.uint16
        lo = 0 if rng.random() < 0.5 else top - top // 8
        ref = rng.integers(lo, top + 1, size=(f, h, stride)).astype(dt)
        dis = rng.integers(0, top + 1, size=(f, h, stride)).astype(dt)
        ref[:, :, w:] = top
        dis[:, :, w:] = top
        batches.append((dev(ref), dev(dis), bpc, w, out_for(f)))
        want.append((n, ref, dis, bpc, w))
    torch.cuda.synchronize()
    say("[gpu] pipe random: 40 batches, seed 20261202")
    run(api, batches, st)
    for (n, ref, dis, bpc, w), b in zip(want, batches):
        emom, eps = orc.frames(ref, dis, bpc, w=w)
        g = b[4].cpu().numpy()
        assert (bits(g[:, :4]) == bits(emom)).all() and (bits(g[:, 4:]) == bits(eps)).all(), (
            n, ref.shape, bpc, w, g, emom, eps)
