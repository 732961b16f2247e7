"""HIP path vs the oracle, bit for bit (needs an MI355X).

Every comparison is ``==`` on the 64-bit patterns of the doubles: the
float_moment and float_psnr outputs must be the CPU loop's own bits
(ADR-1497, Consequences; ADR-1499, Consequences: tolerance 0).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import boundary
import oracle
import random_frames
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


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(x):
    return np.asarray(x, dtype=np.float64).view(np.uint64)


def expect(orc, ref, dis, bpc, w):
    return orc.frames(ref, dis, bpc, w=w)


def check_batch(api, orc, ref, dis, bpc, w=None, label=""):
    say(f"[gpu] {label} frames={ref.shape[0]} h={ref.shape[1]} stride={ref.shape[2]} "
        f"w={w} bpc={bpc}")
    mom, ps = api.bef_frames(dev(ref), dev(dis), bpc, w=w)
    emom, eps = expect(orc, ref, dis, bpc, w)
    bad = np.nonzero((bits(mom) != bits(emom)).any(axis=1) | (bits(ps) != bits(eps)).any(axis=1))[0]
    assert bad.size == 0, (
        f"{label}: {bad.size} frames differ; first {bad[0]}: gpu {mom[bad[0]]} {ps[bad[0]]} "
        f"oracle {emom[bad[0]]} {eps[bad[0]]}")
    return mom, ps


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_workload_parity(api, orc, key):
    """Every frame of each of the five workloads."""
    wl = synth.WORKLOADS[key]
    ref, dis = synth.make_frames(key)
    check_batch(api, orc, ref, dis, wl.bpc, w=wl.w, label=wl.name)


def test_workload_units_past_2_53(api, orc):
    """On full-range 16-bit 4K noise every plane's second-moment sum passes
    2^53 and the CPU's rounded sum differs from the exact one (the twins'
    old exact-once result failed on every such frame: ADR-1497, Context)."""
    ref, dis = synth.make_frames(4, frames=4)
    u = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert (u[:, 2] > (1 << 53)).all() and (u[:, 3] > (1 << 53)).all()
    assert (u[:, 4] != u[:, 2]).all() and (u[:, 5] != u[:, 3]).all()
    for f in range(4):
        acc = orc.moment_sums(ref[f], dis[f], 16)
        assert int(np.float64(acc[2]) * 65536.0) == int(u[f, 4])
        assert int(np.float64(acc[3]) * 65536.0) == int(u[f, 5])


@pytest.mark.parametrize("kind", boundary.KINDS)
def test_boundary_frames(api, orc, kind):
    """The pages' boundary frames, both orientations, with the expected
    accumulators of tests/golden/boundary_frames.txt."""
    import oracle_checks
    gold = oracle_checks.load_golden()[kind]
    p = boundary.build(kind)
    z = np.zeros_like(p)
    ref = np.stack([p, z])
    dis = np.stack([z, p])
    check_batch(api, orc, ref, dis, 16, label=f"boundary {kind}")
    u = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert int(u[0, 4]) == gold["moment"] and int(u[1, 5]) == gold["moment"]
    assert int(u[0, 2]) == gold["exact"] and int(u[1, 3]) == gold["exact"]
    for f in range(2):
        d = np.array([u[f, 7]], dtype=np.uint64).view(np.float64)[0]
        assert int(d) == gold["psnr"]


SHAPES = [
    # (w, h, stride, bpc, frames)
    (1, 1, 1, 8, 1),
    (1, 1, 1, 16, 2),
    (7, 3, 7, 10, 3),          # ragged, unaligned rows
    (64, 2, 64, 16, 2),
    (100, 9, 100, 16, 2),      # 200-byte rows: not 16-byte aligned
    (511, 17, 513, 12, 2),     # odd stride
    (512, 5, 512, 16, 1),
    (520, 33, 520, 16, 3),     # one vector tail lane group
    (4100, 3, 4104, 16, 2),    # more than one 512-vector batch per lane
    (176, 144, 192, 8, 2),     # 8-bit with stride padding
    (1000, 37, 1000, 8, 2),    # 8-bit ragged
    (32768, 2, 32768, 16, 1),  # widest row
    (97, 11, 97, 9, 2),        # every bit depth from 9 to 15
    (130, 7, 132, 11, 2),
    (256, 5, 256, 13, 2),
    (300, 6, 304, 14, 2),
    (33, 40, 40, 15, 3),
]


@pytest.mark.parametrize("w,h,stride,bpc,frames", SHAPES)
def test_shapes(api, orc, w, h, stride, bpc, frames):
    ref, dis = synth.uniform_planes(w * 7 + h, frames, h, w, stride, bpc)
    check_batch(api, orc, ref, dis, bpc, w=w, label=f"shape {w}x{h}/{stride}")


@pytest.mark.parametrize("bpc", [8, 16])
def test_most_frames(api, orc, bpc):
    """The largest batch, 65535 frames (tiny ones: 3x2, rows not aligned),
    every frame against the oracle."""
    ref, dis = synth.uniform_planes(65535 + bpc, 65535, 2, 3, 3, bpc)
    check_batch(api, orc, ref, dis, bpc, w=3, label=f"65535 frames bpc {bpc}")


def test_tallest_plane_past_2_53(api, orc):
    """The tallest plane, h = 32768 (w = 128), with high content so that
    the second-moment sums pass 2^53 late in the plane."""
    rng = np.random.Generator(np.random.PCG64(32768))
    ref = rng.integers(56000, 65536, size=(1, 32768, 128)).astype(np.uint16)
    small = rng.random(size=ref.shape) < 0.05
    ref[small] = rng.integers(0, 4096, size=int(small.sum())).astype(np.uint16)
    dis = rng.integers(0, 65536, size=ref.shape).astype(np.uint16)
    units = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert (units[:, 2] > 1 << 53).all() and (units[:, 4] != units[:, 2]).all()
    check_batch(api, orc, ref, dis, 16, label="128x32768")


CONSTANTS = [(0, 0), (65535, 0), (0, 65535), (65535, 65535), (1, 0), (4095, 4094)]


def test_constant_frames(api, orc):
    """Degenerate 16-bit 3840x2160 frames of one value per plane: zeros,
    the top codeword (every term 0xFFFE0000; the sum crosses 2^53 and 2^54
    with no rounding, since every term is a multiple of 2^17), ones, and
    the largest odd exact square against its neighbour."""
    ref = np.stack([np.full((2160, 3840), r, np.uint16) for r, _ in CONSTANTS])
    dis = np.stack([np.full((2160, 3840), d, np.uint16) for _, d in CONSTANTS])
    check_batch(api, orc, ref, dis, 16, label="constant frames")
    u = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert int(u[1, 2]) == 3840 * 2160 * 0xFFFE0000 == int(u[1, 4])
    assert int(u[0, 2]) == 0 and int(u[0, 7]) == 0


def test_single_frame_entry_points(api, orc):
    wl = synth.WORKLOADS[3]
    ref, dis = synth.make_frames(3, frames=1)
    r, d = dev(ref[0]), dev(dis[0])
    m = api.moment_frame(r, d, 12, w=wl.w)
    p = api.psnr_noise(r, d, 12, w=wl.w)
    assert bits(m).tolist() == bits(orc.moment_frame(ref[0], dis[0], 12, w=wl.w)).tolist()
    assert bits(p).tolist() == bits(orc.psnr_noise(ref[0], dis[0], 12, w=wl.w)).tolist()


def test_single_output_calls_run_their_walk_only(api, orc):
    """moment_frame runs no noise walk and psnr_noise no moment walk (nor
    plan or row pairs), on frames past 2^53 and past 2^55, with the
    oracle's bits."""
    for key in (5, 6):
        wl = synth.WORKLOADS[key]
        ref, dis = synth.make_frames(key, frames=1)
        r, d = dev(ref[0]), dev(dis[0])
        say(f"[gpu] single-output calls on workload {key}")
        m = api.moment_frame(r, d, 16)
        assert api.bef_walk_paths()[0, 2] == 4, api.bef_walk_paths()
        assert (api.bef_walk_paths()[0, :2] != 4).all()
        p = api.psnr_noise(r, d, 16)
        assert (api.bef_walk_paths()[0, :2] == 4).all() and api.bef_walk_paths()[0, 2] != 4
        assert bits(m).tolist() == bits(orc.moment_frame(ref[0], dis[0], 16, w=wl.w)).tolist()
        assert bits(p).tolist() == bits(orc.psnr_noise(ref[0], dis[0], 16, w=wl.w)).tolist()
        mom, ps = api.bef_frames(r[None], d[None], 16)
        assert (api.bef_walk_paths() != 4).all()
        assert bits(mom[0]).tolist() == bits(m).tolist() and bits(ps[0]).tolist() == bits(p).tolist()


DEBUG = [1, 2, 4, 8, 16, 32, 1 | 16, 2 | 32, 8 | 32, 32 | 64]


@pytest.mark.parametrize("flags", DEBUG)
def test_debug_paths_same_bits(api, orc, flags):
    """Wrong plans, no plans, terms only, forced rounding, no stretches, no
    closed form, row pairs in many small dispatches: every path must give
    the CPU's bits (ADR-1497, Decision: a plan, right or wrong, only
    changes which increments are used)."""
    r4, d4 = synth.make_frames(4, frames=2)
    r5, d5 = synth.make_frames(5, frames=1)
    b = boundary.build("b53p3")
    ref = np.concatenate([r4, r5, b[None]])
    dis = np.concatenate([d4, d5, np.zeros_like(b)[None]])
    old = api.bef_debug_set(flags)
    try:
        check_batch(api, orc, ref, dis, 16, label=f"debug {flags}")
    finally:
        api.bef_debug_set(old)


def test_past_2_55_8k_noise(api, orc):
    """16-bit 7680x4320 noise crosses the binades of 2^53, 2^54 and 2^55
    (ADR-1497, Consequences: 4 of 4 such frames identical)."""
    ref, dis = synth.uniform_planes(8000, 2, 4320, 7680, 7680, 16)
    check_batch(api, orc, ref, dis, 16, label="8k noise")


@pytest.mark.parametrize("flags", [1, 2, 1 | 16, 2 | 32, 32 | 64])
def test_8k_noise_debug_paths(api, orc, flags):
    """8K noise (past 2^55) under wrong plans, no plans, no stretches, no
    closed forms and split pair dispatches, each of which sends the planes
    to the general walk: its every path gives the CPU's bits."""
    ref, dis = synth.uniform_planes(8000, 1, 4320, 7680, 7680, 16)
    old = api.bef_debug_set(flags)
    try:
        check_batch(api, orc, ref, dis, 16, label=f"8k noise, debug {flags}")
    finally:
        api.bef_debug_set(old)


def test_noise_past_2_55_tall(api, orc):
    """A 7680x4608 frame of high ref against low dis: the noise passes 2^55
    on a plane taller than one chunk of rows (4352 rows), so the noise runs
    chunk by chunk past 2^53, and both moments pass 2^55."""
    rng = np.random.Generator(np.random.PCG64(7655))
    ref = rng.integers(48000, 65536, size=(1, 4608, 7680)).astype(np.uint16)
    dis = rng.integers(0, 16000, size=(1, 4608, 7680)).astype(np.uint16)
    u = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert int(u[0, 6]) > 1 << 55
    check_batch(api, orc, ref, dis, 16, label="7680x4608 noise past 2^55")


def test_past_2_55_4096x2560(api, orc):
    """A 4096x2560 frame past 2^55 (ADR-1497, Consequences): near-maximum
    content with small codewords mixed in, so that the binade of 2^55 holds
    ties; both planes' exact sums pass 2^55 (checked here with numpy)."""
    rng = np.random.Generator(np.random.PCG64(2555))
    ref = np.stack([synth.nearmax_plane(rng, 2560, 4096, 60000) for _ in range(2)]).astype(np.uint16)
    dis = np.stack([synth.nearmax_plane(rng, 2560, 4096, 58000) for _ in range(2)]).astype(np.uint16)
    for p in (ref, dis):
        sq = p.astype(np.float32) * p.astype(np.float32)  # float multiply, RNE
        assert (sq.astype(np.int64).sum(axis=(1, 2)) > 1 << 55).all()
    check_batch(api, orc, ref, dis, 16, label="4096x2560 past 2^55")


def binade55_plane(k: int, wide: bool = False):
    """Seeded near-maximum 16-bit plane (a fraction of small codewords, some
    of whose squares tie in the binade of 2^55) of width 3500-4096 (wide:
    4097-8192, on its own seeds) and at most 4352 rows, its exact sum in
    the binade of 2^55; k == 5: its last 15% of rows are zeros."""
    seed = [0xBEF, 5556 if wide else 5555, k]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    w = int(rng.integers(4097, 8193) if wide else rng.integers(3500, 4097))
    pad = int(rng.choice([0, 0, 3, 8]))
    lo = int(rng.integers(50000, 62000))
    small = float(rng.choice([0.0, 0.02, 0.05, 0.2]))
    target = float(rng.uniform(55.05, 55.9))
    sq = np.arange(65536, dtype=np.float32) ** 2  # float squares of every codeword
    mean = (1 - small) * float(sq[lo:].mean()) + small * float(sq[:8192].mean())
    h = min(4352, int(2 ** target / (w * mean)))
    body = synth.nearmax_plane(rng, h, w, lo, small)
    if k == 5:
        body[int(h * 0.85):] = 0
    ref = np.full((1, h, w + pad), 0xFFFF, np.uint16)
    ref[0, :, :w] = body
    dis = np.full_like(ref, 0xFFFF)
    dis[0, :, :w] = 0 if k % 2 else rng.integers(0, 65536, size=(h, w))
    return ref, dis, w


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("k", range(6))
def test_fast_walk_in_the_binade_of_2_55(api, orc, k, wide):
    """Planes whose exact sum lies in [2^55, 2^56), at most 8192 wide (the
    wide cases stage a crossing row in two rounds of loads) and 4352 tall,
    take the fast walk's seven-edge form (rows across 2^53, 2^54 and 2^55
    walked term-wise, the stretch inside the binade of 2^55 as the rows'
    pairs joined in order, a crossing row's part in that binade from its
    lanes' runs) and give the oracle's bits; case 5 ends in rows of zeros
    past 2^55 (ADR-1497, Decision: the walk's steps)."""
    ref, dis, w = binade55_plane(k, wide)
    u = api.bef_frames_units(dev(ref), dev(dis), 16, w=w)
    assert (1 << 55) <= int(u[0, 2]) < (1 << 56), int(u[0, 2])
    check_batch(api, orc, ref, dis, 16, w=w, label=f"binade 55 plane {k}")
    assert int(api.bef_walk_paths()[0, 0]) == 1  # the ref plane's moments: the fast walk


def test_past_2_53_2560x1440_16bit(api, orc):
    """A 16-bit 2560x1440 frame past 2^53, the size on which the twins'
    rounded-once result was measured off (ADR-1497, Context).  High content
    fills the ref plane to about 2^53.2 units, and one sample in ten is a
    small codeword whose odd square ties past 2^53 (squares of codewords of
    2^15.5 and more are multiples of 2^7 and add exactly there); dark dis
    content puts the noise past 2^53 as well; rows are padded to 2624 samples of
    0xFFFF that must never be read."""
    rng = np.random.Generator(np.random.PCG64(2560))
    ref = np.full((2, 1440, 2624), 0xFFFF, dtype=np.uint16)
    dis = np.full_like(ref, 0xFFFF)
    body = rng.integers(46000, 65536, size=(2, 1440, 2560))
    small = rng.random(size=body.shape) < 0.1  # odd squares: ties past 2^53
    body[small] = rng.integers(0, 4096, size=int(small.sum()))
    ref[:, :, :2560] = body
    dis[:, :, :2560] = rng.integers(0, 8000, size=(2, 1440, 2560))
    units = api.bef_frames_units(dev(ref), dev(dis), 16, w=2560)
    assert (units[:, 2] > 1 << 53).all() and (units[:, 4] != units[:, 2]).any()
    assert (units[:, 6] > 1 << 53).all()
    check_batch(api, orc, ref, dis, 16, w=2560, label="2560x1440 16-bit past 2^53")


@pytest.mark.parametrize("k", range(random_frames.N_GPU_CASES))
def test_random_crossings(api, orc, k):
    """Seeded random planes whose sum crosses 2^53 or 2^54 at a random row
    and column, with random width, padding, bit depth, tail and dis."""
    ref, dis, w, bpc, label = random_frames.case(k)
    check_batch(api, orc, ref[None], dis[None], bpc, w=w, label=label)


@pytest.mark.parametrize("w,stride,path", [(7680, 7680, 1), (8192, 8192, 1), (8190, 8193, 1),
                                           (8200, 8200, 2), (10000, 10003, 2)])
def test_wide_rows_past_2_53(api, orc, w, stride, path):
    """Full-range noise, 1100 rows, crosses 2^53 inside a wide row.  Rows of
    up to 8192 samples take the fast walk, which stages a crossing row in
    LDS in two rounds of 16-byte loads, or sample by sample when the row is
    not whole 16-byte chunks (8190 samples, odd stride); wider rows take
    the general walk, which stages them with the whole block."""
    ref, dis = synth.uniform_planes(7681 + w, 1, 1100, w, stride, 16)
    units = api.bef_frames_units(dev(ref), dev(dis), 16, w=w)
    assert (units[:, 2] > 1 << 53).all()
    check_batch(api, orc, ref, dis, 16, w=w, label=f"{w}x1100 stride {stride}")
    assert (api.bef_walk_paths()[:, :2] == path).all(), api.bef_walk_paths()


@pytest.mark.parametrize("hi,lo_e,hi_e", [(46000, 54, 55), (65536, 55, 56)])
def test_fast_walk_at_its_largest_plane(api, orc, hi, lo_e, hi_e):
    """16-bit 8192x4352 noise, the widest rows and the most rows the fast
    walk takes (every staged row and every chunk of row sums full): U[0,
    45999] sums into the binade of 2^54 (five edges), the full range into
    that of 2^55 (seven edges, the rows' pairs in that binade).  Both
    moment blocks take the fast walk and give the oracle's bits."""
    ref, dis = synth.uniform_planes(8192 + hi, 1, 4352, 8192, 8192, 16, hi=hi)
    units = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert ((units[:, 2:4] >= 1 << lo_e) & (units[:, 2:4] < 1 << hi_e)).all(), units[:, 2:4]
    check_batch(api, orc, ref, dis, 16, label=f"8192x4352 U[0,{hi - 1}]")
    assert (api.bef_walk_paths()[:, :2] == 1).all(), api.bef_walk_paths()


@pytest.mark.parametrize("h", [4352, 4353])
def test_one_chunk_of_rows_past_2_53(api, orc, h):
    """2048-wide full-range noise past 2^53 (below 2^55) in a plane of
    exactly as many rows as the walk holds in LDS (4352: the fast path with
    its most rows per thread) and in one row more (the general walk)."""
    ref, dis = synth.uniform_planes(h, 1, h, 2048, 2048, 16)
    units = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert (units[:, 2] > 1 << 53).all() and (units[:, 2] < 1 << 55).all()
    check_batch(api, orc, ref, dis, 16, label=f"2048x{h}")
    # at 4352 rows a lane of the fast walk owns 72 rows (more than a wave
    # scans at once): the edges are still found and the fast path holds
    paths = api.bef_walk_paths()
    want = 1 if h <= 4352 else 2
    assert (paths[:, :2] == want).all(), paths


def test_walk_paths(api):
    """Which path each walk block takes: the fast walk on 16-bit
    3840x2160 frames (full and half range) and on 4096x2560 frames whose
    sums lie in the binade of 2^55 and on 7680x4320 noise (its seven-edge
    form), exact sums only on 10-bit frames that cannot pass 2^53, and the
    general walk under a test flag."""
    cases = [(4, 2, [[1, 1, 1]]), (5, 2, [[1, 1, 1]]), (2, 2, [[0, 0, 0]]), (6, 1, [[1, 1, 1]]),
             (7, 1, [[1, 1, 1]])]
    for key, nf, want in cases:
        ref, dis = synth.make_frames(key, frames=nf)
        say(f"[gpu] walk paths of workload {key}")
        api.bef_frames(dev(ref), dev(dis), synth.WORKLOADS[key].bpc, w=synth.WORKLOADS[key].w)
        paths = api.bef_walk_paths()
        assert paths.shape == (nf, 3) and (paths == np.array(want)).all(), (key, paths)
    ref, dis = synth.make_frames(4, frames=1)
    old = api.bef_debug_set(api.DBG_PLAN_WRONG)
    try:
        api.bef_frames(dev(ref), dev(dis), 16)
    finally:
        api.bef_debug_set(old)
    assert (api.bef_walk_paths() == np.array([[2, 2, 3]])).all(), api.bef_walk_paths()


def test_tall_plane_past_2_53(api, orc):
    """1024x8192 full-range noise: more rows than the walk holds in LDS."""
    ref, dis = synth.uniform_planes(8193, 1, 8192, 1024, 1024, 16)
    units = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert (units[:, 2] > 1 << 53).all()
    check_batch(api, orc, ref, dis, 16, label="1024x8192")


def test_letterbox_rows_of_zeros_after_2_53(api, orc):
    """Bright rows take the exact sum to 2^53 + 5000, then rows of zeros (a
    black band) follow while the sum sits within the walk's margin of the
    edge: every such row is checked against the actual running sum."""
    ref = np.zeros((2, 2160, 3840), np.uint16)
    for f in range(2):
        boundary._fill_to(ref[f].reshape(-1), 0, (1 << 53) + 5000, 40000, 65536,
                          np.random.Generator(np.random.PCG64(1653 + f)), False)
    dis = synth.uniform_planes(1653, 2, 2160, 3840, 3840, 16)[1]
    units = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert (units[:, 2] == (1 << 53) + 5000).all()
    check_batch(api, orc, ref, dis, 16, label="letterbox")


def test_noise_past_2_54(api, orc):
    """ref high, dis low: the PSNR noise passes 2^54 units below 2^55, so its
    row adds round in the binades of 2^53 and 2^54 (ADR-1499, Decision:
    every rounding past 2^53, ties included, is the CPU's)."""
    rng = np.random.Generator(np.random.PCG64(5454))
    ref = rng.integers(48000, 65536, size=(2, 2160, 3840)).astype(np.uint16)
    dis = rng.integers(0, 16000, size=(2, 2160, 3840)).astype(np.uint16)
    units = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert ((units[:, 6] >= 1 << 54) & (units[:, 6] < 1 << 55)).all(), units[:, 6]
    check_batch(api, orc, ref, dis, 16, label="noise past 2^54")


@pytest.mark.parametrize("mode", synth.WIDEN_MODES)
def test_widened_smooth_content(api, orc, mode):
    """Smooth 8-bit content widened to 16 bits three ways (ADR-1497,
    Consequences): by a shift (every square exact past 2^53), by 257 and
    with a dithered low byte (odd squares in a dark band past 2^53).  Four
    frames whose sums fall on both sides of 2^53 units."""
    ref, dis = synth.widened_frames(mode, 4)
    units = api.bef_frames_units(dev(ref), dev(dis), 16)
    assert (units[:, 2] > 1 << 53).any() and (units[:, 2] < 1 << 53).any()
    check_batch(api, orc, ref, dis, 16, label=f"widened {mode}")


def test_async_matches_sync(api, orc):
    import torch
    ref, dis = synth.make_frames(5, frames=3)
    r, d = dev(ref), dev(dis)
    out = torch.zeros((3, 6), dtype=torch.float64, device="cuda")
    api.bef_frames_async(r, d, 16, out)
    torch.cuda.synchronize()
    mom, ps = api.bef_frames(r, d, 16)
    got = out.cpu().numpy()
    assert (bits(got[:, :4]) == bits(mom)).all() and (bits(got[:, 4:]) == bits(ps)).all()


def test_graph_capture_replays(api, orc):
    """bef_frames_async only enqueues kernels once its scratch has grown (no
    allocation, memset or sync), so a caller can capture it in a HIP graph.
    Each replay reads whatever frames the buffers then hold: two frame sets
    alternate, with eager copies and syncs between replays, and every replay
    is checked against the oracle."""
    import torch
    r5, d5 = synth.make_frames(5, frames=2)
    r4, d4 = synth.make_frames(4, frames=2)
    want = {k: expect(orc, r, d, 16, None) for k, (r, d) in {5: (r5, d5), 4: (r4, d4)}.items()}
    R, D = dev(r5), dev(d5)
    out = torch.zeros((2, 6), dtype=torch.float64, device="cuda")
    api.bef_frames_async(R, D, 16, out)  # grows the scratch outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.bef_frames_async(R, D, 16, out)
    torch.cuda.synchronize()
    for n, key in enumerate([4, 5, 4, 5, 5]):
        r, d = (r4, d4) if key == 4 else (r5, d5)
        R.copy_(torch.from_numpy(r))
        D.copy_(torch.from_numpy(d))
        out.fill_(-1.0)
        torch.cuda.synchronize()
        say(f"[gpu] graph replay {n} frames of workload {key}")
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        emom, eps = want[key]
        assert (bits(got[:, :4]) == bits(emom)).all() and (bits(got[:, 4:]) == bits(eps)).all(), n


def test_deterministic(api):
    ref, dis = synth.make_frames(4, frames=2)
    r, d = dev(ref), dev(dis)
    a = api.bef_frames_units(r, d, 16)
    b = api.bef_frames_units(r, d, 16)
    assert (a == b).all()


@pytest.mark.parametrize("key,pinned", [(5, False), (5, True), (3, True), (7, True)])
def test_host_pipeline_matches_device(api, orc, key, pinned):
    """Frames from host memory, streamed through the two device slots (the
    12-bit workload takes four chunks, so both slots are reloaded; the
    4096x2560 near-maximum frames pass 2^55, so each chunk plans and forms
    row pairs), give the same bits as the device entry point and the
    oracle."""
    import torch
    wl = synth.WORKLOADS[key]
    ref, dis = synth.make_frames(key)
    say(f"[gpu] host pipeline workload {key} pinned={pinned}")
    if pinned:
        r, d = torch.from_numpy(ref).pin_memory(), torch.from_numpy(dis).pin_memory()
    else:
        r, d = ref, dis
    hmom, hps = api.bef_frames_host(r, d, wl.bpc, w=wl.w)
    mom, ps = api.bef_frames(dev(ref), dev(dis), wl.bpc, w=wl.w)
    assert (bits(hmom) == bits(mom)).all() and (bits(hps) == bits(ps)).all()
    emom, eps = expect(orc, ref[:2], dis[:2], wl.bpc, wl.w)
    assert (bits(hmom[:2]) == bits(emom)).all() and (bits(hps[:2]) == bits(eps)).all()


def test_host_pipeline_frame_pitch(api, orc):
    """Host frames that are not contiguous (a frame pitch above h * stride)
    are uploaded frame by frame; same bits as the device path."""
    import ctypes
    wl = synth.WORKLOADS[3]
    ref, dis = synth.make_frames(3, frames=5)
    F, h, stride = ref.shape
    gap = 3  # rows of padding between frames
    rbig = np.full((F, h + gap, stride), 0xFFFF, np.uint16)
    dbig = np.full((F, h + gap, stride), 0xFFFF, np.uint16)
    rbig[:, :h] = ref
    dbig[:, :h] = dis
    mom = np.zeros((F, 4), np.float64)
    ps = np.zeros((F, 2), np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = api.lib().bef_frames_host(rbig.ctypes.data, dbig.ctypes.data, wl.w, h, stride,
                                   (h + gap) * stride, F, wl.bpc, 0, mom.ctypes.data_as(dp),
                                   ps.ctypes.data_as(dp))
    assert rc == 0, api.last_error()
    dmom, dps = api.bef_frames(dev(ref), dev(dis), wl.bpc, w=wl.w)
    assert (bits(mom) == bits(dmom)).all() and (bits(ps) == bits(dps)).all()


def test_read_ceiling_diagnostic(api):
    """The read-only diagnostic pass runs on the row pass's shapes, gives
    the same words twice, and rejects rows with no whole 4-byte chunk."""
    import torch
    ref, dis = synth.make_frames(5, frames=2)
    r, d = dev(ref), dev(dis)
    out1 = torch.zeros(2 * ref.shape[1], dtype=torch.int32, device="cuda")
    out2 = torch.ones_like(out1)
    api.bef_read_ceiling(r, d, out1)
    api.bef_read_ceiling(r, d, out2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    buf = torch.zeros(8 * 33 + 1, dtype=torch.uint16, device="cuda")
    odd = buf[1:].view(1, 8, 33)  # contiguous, starts 2 bytes past an aligned address
    with pytest.raises(api.BefError):
        api.bef_read_ceiling(odd, odd, out1, w=32)


def test_bad_arguments(api):
    import torch
    r = torch.zeros((4, 4), dtype=torch.uint16, device="cuda")
    lib = api.lib()
    out = (api.ctypes.c_double * 4)()
    p = r.data_ptr()
    assert lib.moment_frame(p, p, 0, 4, 4, 16, out) == -22
    assert lib.moment_frame(p, p, 4, 0, 4, 16, out) == -22
    assert lib.moment_frame(p, p, 4, 4, 3, 16, out) == -22
    assert lib.moment_frame(p, p, 4, 4, 4, 7, out) == -22
    assert lib.moment_frame(p, p, 40000, 4, 40000, 16, out) == -22
    assert lib.moment_frame(None, p, 4, 4, 4, 16, out) == -22
    host = np.zeros((4, 4), np.uint16)
    assert lib.moment_frame(host.ctypes.data, host.ctypes.data, 4, 4, 4, 16, out) == -22
    assert api.last_error() != ""
    assert lib.moment_frame(p, p, 4, 4, 4, 16, None) == -22
    assert "NULL out" in api.last_error()
    assert lib.psnr_noise(p, p, 4, 4, 4, 16, None) == -22
    assert "NULL out" in api.last_error()


def test_stream_of_the_planes_device(api, orc):
    """A caller's stream on the planes' device is accepted, by the sync,
    async and diagnostic entry points alike."""
    import torch
    ref, dis = synth.make_frames(2, frames=2)
    r, d = dev(ref), dev(dis)
    s = torch.cuda.Stream()
    mom, ps = api.bef_frames(r, d, 10, w=synth.WORKLOADS[2].w, stream=s)
    emom, eps = expect(orc, ref, dis, 10, synth.WORKLOADS[2].w)
    assert (bits(mom) == bits(emom)).all() and (bits(ps) == bits(eps)).all()
    out = torch.zeros((2, 6), dtype=torch.float64, device="cuda")
    api.bef_frames_async(r, d, 10, out, w=synth.WORKLOADS[2].w, stream=s)
    s.synchronize()
    got = out.cpu().numpy()
    assert (bits(got[:, :4]) == bits(emom)).all() and (bits(got[:, 4:]) == bits(eps)).all()


def test_timing_counters(api):
    """Per-kernel timing counts each timed launch once, and a reset clears
    every counter, the read-ceiling one included."""
    import torch
    ref, dis = synth.make_frames(4, frames=2)
    r, d = dev(ref), dev(dis)
    cout = torch.zeros(2 * ref.shape[1], dtype=torch.int32, device="cuda")
    api.bef_timing_enable(True)
    try:
        api.bef_timing_reset()
        for _ in range(3):
            api.bef_frames(r, d, 16)
            api.bef_read_ceiling(r, d, cout)
        torch.cuda.synchronize()
        counts = {k: api.bef_timing_read(k) for k in ("rows", "walk", "ceiling")}
        assert all(n == 3 and ms > 0 for ms, n in counts.values()), counts
        api.bef_timing_reset()
        assert all(api.bef_timing_read(k) == (0.0, 0) for k in api.KERNELS), \
            {k: api.bef_timing_read(k) for k in api.KERNELS}
    finally:
        api.bef_timing_enable(False)
        api.bef_timing_reset()
