"""The C-ABI library and the host emulation on the CPU (no GPU call).

- libbef.so loads (it links the HIP runtime, which loads without a GPU) and
  exports every symbol include/bef.h declares, and no test entry point.
- The host emulation library (host_emu.h, built from host_emu.cpp with the
  kernels' step header and shape constants) runs the kernels' decomposition
  serially: its one-term step is checked against the hardware double add,
  its run pairs against brute force, and its walks against the oracle, with
  real plans and with the test flags' wrong or missing plans (the pages' own
  host test does the same for their twins: ADR-1497, Decision).
- Breaks planted in the step header (ADR-1497, Consequences lists most of
  them) and in the group step of a crossing row each make the emulation
  disagree with the oracle.
"""
from __future__ import annotations

import ctypes
import functools
import math
import os
import re

import numpy as np
import pytest

import boundary
import checkers
import oracle
import random_frames
from bit_exact_frame_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bef.h")


@pytest.fixture(scope="module")
def api():
    import emu
    return emu.Emu()


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def declared(header):
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    return sorted({n for n in names if n not in ("defined",)})


def test_every_declared_symbol_is_exported():
    """libbef.so exports every entry point of include/bef.h and none of the
    test entry points; the emulation library exports those of host_emu.h."""
    import emu
    from bit_exact_frame_amd import api
    decl = declared(HEADER)
    assert "moment_frame" in decl and "psnr_noise" in decl and "bef_frames" in decl
    assert "bef_frames_noalloc" in decl
    lib = ctypes.CDLL(api.LIB_PATH)
    missing = [n for n in decl if not hasattr(lib, n)]
    assert not missing, missing
    test_decl = declared(emu.HEADER)
    assert test_decl and all(n.startswith("bef_host_") for n in test_decl), test_decl
    assert not [n for n in test_decl if hasattr(lib, n)]
    em = emu.Emu()
    assert not [n for n in test_decl if not hasattr(em.lib, n)]


# --------------------------------------------------------------- one step --

def test_one_term_step_against_double_add(api):
    """fl64(S + t) in units for 400 000 random (S, t): S a double holding an
    integer between 2^50 and 2^58, t below 2^32."""
    rng = np.random.Generator(np.random.PCG64(53))
    n = 400_000
    e = rng.integers(50, 58, size=n)
    mant = rng.integers(1 << 52, 1 << 53, size=n, dtype=np.int64)
    s = np.ldexp(mant.astype(np.float64), (e - 52).astype(np.int64))
    s = np.maximum(np.round(s), 1.0)
    t = rng.integers(0, 1 << 32, size=n, dtype=np.int64)
    want = (s + t.astype(np.float64))  # IEEE double add, round to nearest even
    f = api.lib.bef_host_rne53_add
    for k in range(n):
        assert f(int(s[k]), int(t[k])) == int(want[k]), (int(s[k]), int(t[k]))


def test_one_term_step_boundary_pairs(api):
    """Every pair around the binade edges 2^53..2^58 and around the ties."""
    f = api.rne53_add
    for e in range(53, 59):
        u = 1 << (e - 52)
        for base in (1 << e, (1 << e) - u // 2 if u > 1 else (1 << e) - 1, (1 << (e + 1)) - u):
            base = int(float(base))  # a value the double can hold
            for t in {0, 1, u // 2 - 1, u // 2, u // 2 + 1, u - 1, u, u + 1, 3 * u // 2,
                      (1 << 32) - 1}:
                if t < 0:
                    continue
                assert f(base, t) == int(float(base) + float(t)), (e, base, t)
    for s in range((1 << 53) - 4, (1 << 53) + 1):
        for t in range(0, 8):
            assert f(s, t) == int(float(s) + float(t)), (s, t)


# --------------------------------------------------------------- run pair --

def brute_pair(terms, e):
    """Both starting parities of binade e, term by term with the integer
    IEEE step, from a start well inside the binade."""
    u = 1 << (e - 52)
    out = []
    for p in (0, 1):
        s0 = (1 << e) + (1 << (e - 2)) + p * u
        s = s0
        for t in terms:
            s = checkers.rne(s + int(t), 53)
        assert s < (1 << (e + 1))
        out.append(s - s0)
    return out


def test_run_pair_brute_force(api):
    rng = np.random.Generator(np.random.PCG64(7))
    tt = checkers.t_table()
    for trial in range(400):
        e = int(rng.integers(53, 60))
        n = int(rng.integers(0, 80))
        if trial % 2:
            x = rng.integers(0, 65536, size=n)
        else:  # small codewords: dense ties and parity flips
            x = rng.integers(0, 9000, size=n)
        terms = tt[x].astype(np.uint32)
        assert api.run_pair(terms, e) == brute_pair(terms.tolist(), e), (e, n)


def test_run_pair_long_runs_stay_in_their_binade(api):
    """Runs of up to 2^15 terms, the largest a row holds, at the top of the
    term range: the double-add pair still equals the brute-force integer
    fold in binades 53 to 62 (every add stays inside the binade)."""
    rng = np.random.Generator(np.random.PCG64(15))
    tt = checkers.t_table()
    for e in (53, 55, 58, 62):
        for n in (4096, 32768):
            x = rng.integers(60000, 65536, size=n)
            small = rng.random(n) < 0.1  # small codewords: odd terms, ties
            x[small] = rng.integers(0, 4096, size=int(small.sum()))
            terms = tt[x].astype(np.uint32)
            assert api.run_pair(terms, e) == brute_pair(terms.tolist(), e), (e, n)


def test_run_pair_first_tie(api):
    """Binades 55 to 60: the two moves of a run differ only from its first
    tie on (a term whose remainder modulo u is u/2).  Before it the even and
    odd starts take the same steps, u apart; the tie rounds both to an even
    multiple of u, one down and one up, so from then on they are equal or 2u
    apart and take the same steps again.  So the moves are equal when no term
    is a tie, and differ by exactly u otherwise; the direction is that of the
    even start's parity at the first tie (ADR-1497, Decision: a run of terms
    is an even-start and an odd-start increment).  Checked on runs with no
    tie (terms that are multiples of u), with ties only in the last term, and
    with dense ties, against the double-add pair and the integer fold."""
    rng = np.random.Generator(np.random.PCG64(55))
    tt = checkers.t_table().astype(np.int64)
    for trial in range(600):
        e = int(rng.integers(55, 61))
        u = 1 << (e - 52)
        n = int(rng.integers(1, 120))
        kind = trial % 3
        if kind == 0:  # no tie: every term a multiple of u
            x = rng.integers(0, 65536, size=n)
            terms = tt[x] & ~(u - 1)
        elif kind == 1:  # one tie, at the end
            x = rng.integers(0, 65536, size=n)
            terms = tt[x] & ~(u - 1)
            terms[-1] = terms[-1] | (u // 2)
        else:  # small codewords: ties all along
            terms = tt[rng.integers(0, 9000, size=n)]
        terms = terms.astype(np.uint32)
        tl = [int(t) for t in terms]
        a0, a1 = brute_pair(tl, e)
        assert api.run_pair(terms, e) == [a0, a1], (e, n, kind)
        ties = [k for k, t in enumerate(tl) if t % u == u // 2]
        if not ties:
            assert a1 == a0, (e, n, kind)
            continue
        # the even start's position (in units of u) just before the first tie
        pos = ((1 << e) + (1 << (e - 2))) // u
        for t in tl[: ties[0]]:
            pos += (t + u // 2) // u  # no tie here: the nearest multiple
        q = tl[ties[0]] // u
        # the even start rounds down when pos + q is even, the odd start
        # (one further) then rounds up: one u more
        assert a1 - a0 == (u if (pos + q) % 2 == 0 else -u), (e, n, kind)


def test_closed_form_premise():
    """Every float square in units is 0 or 1 modulo 4, and odd exactly when
    the codeword is odd and below 4096 (exhaustive over 16-bit samples)."""
    tt = checkers.t_table().astype(np.int64)
    x = np.arange(65536)
    assert set(np.unique(tt % 4).tolist()) <= {0, 1}
    assert ((tt % 2 == 1) == ((x % 2 == 1) & (x < 4096))).all()
    assert (tt[1::2][: 2048] % 8 == 1).all()  # odd squares are 1 mod 8


def test_closed_form_against_runs(api):
    """Binades of 2^53 and 2^54: the row pair from (exact sum, odd count)
    equals the pair of the same terms formed by the two-trajectory fold."""
    rng = np.random.Generator(np.random.PCG64(11))
    tt = checkers.t_table()
    for trial in range(300):
        n = int(rng.integers(0, 3000))
        x = rng.integers(0, 65536 if trial % 3 else 6000, size=n)
        terms = tt[x].astype(np.uint32)
        E = int(terms.astype(np.uint64).sum())
        c = int((terms & 1).sum())
        assert api.run_pair(terms, 53) == [E - c, E - c + (2 if c else 0)]
        assert api.run_pair(terms, 54) == [E - c, E - c]


# ------------------------------------------------- host emulation vs oracle --

@functools.lru_cache(maxsize=None)
def planes():
    """(name, plane) cases: both planes of a full-range and a half-range 4K
    frame, the boundary frames, 8K noise (binades 53..55) and a 4096x2560
    frame past 2^55 with small codewords mixed in."""
    out = []
    r4, d4 = synth.make_frames(4, frames=1)
    r5, d5 = synth.make_frames(5, frames=1)
    out += [("c4 ref", r4[0]), ("c4 dis", d4[0]), ("c5 ref", r5[0])]
    out += [(f"boundary {k}", boundary.build(k)) for k in boundary.KINDS]
    r8, _ = synth.uniform_planes(8000, 1, 4320, 7680, 7680, 16)
    out.append(("8k noise", r8[0]))
    rng = np.random.Generator(np.random.PCG64(2555))
    p = synth.nearmax_plane(rng, 2560, 4096, 60000).astype(np.uint16)
    sq = p.astype(np.float32) * p.astype(np.float32)  # float multiply, RNE
    assert int(sq.astype(np.int64).sum()) > 1 << 55
    out.append(("4096x2560 mixed", p))
    return out


@functools.lru_cache(maxsize=None)
def oracle_units(name):
    orc = oracle.Oracle()
    p = dict(planes())[name]
    z = np.zeros_like(p)
    acc = orc.moment_sums(p, z, 16)
    return int(math.ldexp(acc[0], 8)), int(math.ldexp(acc[2], 16))


FLAGS = [0, 1, 2, 8, 16, 32, 1 | 16 | 32, 2 | 32]


@pytest.mark.parametrize("flags", FLAGS)
def test_host_emulation_matches_oracle(api, flags):
    for name, p in planes():
        s1, s2 = oracle_units(name)
        got = api.plane_units(p, 16, dbg=flags)
        assert got[0] == s1, name
        assert got[1] == int(checkers.terms_moment(p).sum(dtype=np.uint64)), name
        assert got[2] == s2, (name, flags, got[2], s2)


def test_host_emulation_terms_only(api):
    """Rows that leave the plan go term by term (a slow path: two frames)."""
    for name, p in planes()[:4]:
        assert api.plane_units(p, 16, dbg=4 | 2)[2] == oracle_units(name)[1], name


@functools.lru_cache(maxsize=None)
def letterbox_plane():
    """Exact sum 2^53 + 5000 from bright samples, then rows of zeros."""
    p = np.zeros((2160, 3840), np.uint16)
    boundary._fill_to(p.reshape(-1), 0, (1 << 53) + 5000, 40000, 65536,
                      np.random.Generator(np.random.PCG64(1653)), False)
    return p


@functools.lru_cache(maxsize=None)
def past_2_56_plane():
    """5120x4096 near-maximum content (one sample in twenty small): the
    exact sum passes 2^56, beyond the fast path."""
    rng = np.random.Generator(np.random.PCG64(2556))
    return synth.nearmax_plane(rng, 4096, 5120, 60000).astype(np.uint16)


@functools.lru_cache(maxsize=None)
def largest_fast_plane():
    """16-bit 8192x4352 full-range noise: the widest rows and the most rows
    the device's fast walk takes, summed into the binade of 2^55."""
    r, _ = synth.uniform_planes(8192 + 65536, 1, 4352, 8192, 8192, 16)
    return r[0]


def test_fast_emulation_matches_oracle(api):
    """The fast path's decisions (threshold edges, closed forms, rows and
    terms at an edge, and for sums in the binade of 2^55 the seven-edge form
    with its pairs joined in that binade) give the oracle's sum on every
    plane below 2^56 (8K noise, the 4096x2560 plane and the 8192x4352 plane
    reach the binade of 2^55), and hand the planes past 2^56 to the general
    walk."""
    cases = list(planes()) + [("letterbox", letterbox_plane()), ("past 2^56", past_2_56_plane()),
                              ("8192x4352", largest_fast_plane())]
    seen55 = 0
    for name, p in cases:
        got = api.fast_units(p, 16)
        exact = int(checkers.terms_moment(p).sum(dtype=np.uint64))
        assert got[2] == exact, name
        if exact >= 1 << 56:
            assert got[0] == 0, name
            continue
        seen55 += exact >= 1 << 55
        if name in ("letterbox", "8192x4352"):
            acc = oracle.Oracle().moment_sums(p, np.zeros_like(p), 16)
            want = int(math.ldexp(acc[2], 16))
        else:
            want = oracle_units(name)[1]
        assert got[0] == 1 and got[1] == want, (name, got, want)
    assert seen55 == 3
    assert int(checkers.terms_moment(past_2_56_plane()).sum(dtype=np.uint64)) >= 1 << 56


@pytest.mark.parametrize("k", range(random_frames.N_CASES))
def test_emulation_random_crossings(api, orc, k):
    """The general walk and the fast path's decisions, emulated on the host,
    give the oracle's sums on seeded random planes that cross 2^53 or 2^54
    at a random row and column; the fast noise too."""
    ref, dis, w, bpc, label = random_frames.case(k)
    acc = orc.moment_sums(ref, dis, bpc, w=w)
    want = int(math.ldexp(acc[2], 2 * (bpc - 8)))
    exact = int(checkers.terms_moment(ref[:, :w]).sum(dtype=np.uint64))
    got = api.plane_units(ref, bpc, w=w)
    assert got[1] == exact and got[2] == want, (label, got, want)
    fast = api.fast_units(ref, bpc, w=w)
    assert fast[0] == 1 and fast[1] == want and fast[2] == exact, (label, fast, want)
    fn = api.fast_noise(ref, dis, bpc, w=w)
    noise = orc.psnr_sum(ref, dis, bpc, w=w)
    assert fn[0] == 1, label
    assert np.array([fn[1]], np.uint64).view(np.float64)[0] == math.ldexp(noise, 2 * (bpc - 8)), label


@functools.lru_cache(maxsize=None)
def noise_pairs():
    """Frame pairs whose noise rounds: half-range (binade of 2^53) and a
    high/low pair past 2^54."""
    r5, d5 = synth.make_frames(5, frames=1)
    rng = np.random.Generator(np.random.PCG64(5454))
    hi = rng.integers(48000, 65536, size=(2160, 3840)).astype(np.uint16)
    lo = rng.integers(0, 16000, size=(2160, 3840)).astype(np.uint16)
    return [("c5", r5[0], d5[0]), ("past 2^54", hi, lo)]


def test_fast_noise_emulation_matches_oracle(api, orc):
    for name, r, d in noise_pairs():
        got = api.fast_noise(r, d, 16)
        noise = orc.psnr_sum(r, d, 16)
        assert got[0] == 1, name
        assert np.array([got[1]], np.uint64).view(np.float64)[0] == math.ldexp(noise, 16), name


def test_host_noise_matches_oracle(api, orc):
    for key in (4, 5):
        r, d = synth.make_frames(key, frames=1)
        bits, ex = api.noise_units(r[0], d[0], 16)
        noise = orc.psnr_sum(r[0], d[0], 16)
        assert np.array([bits], np.uint64).view(np.float64)[0] == math.ldexp(noise, 16)
        assert ex == checkers.psnr_units(r[0], d[0])[1]


# ------------------------------------------------------ row kernel shape --

# (bytes per load, slots per group) the row kernel's launcher instantiates
LAUNCHED = {(8, 4), (8, 5), (8, 8), (8, 15), (4, 4), (4, 5), (4, 8), (4, 15), (0, 1)}


def test_load_shape_choice(api):
    """For many widths and alignments the host picks 8-byte loads whenever
    the rows allow them (else 4-byte ones), a shape the launcher has a kernel
    for, the fewest idle lane slots for that width, and on a tie the larger
    group."""
    rng = np.random.Generator(np.random.PCG64(44))
    widths = [1, 2, 3, 4, 7, 8, 64, 100, 176, 511, 512, 520, 1000, 1280, 1920, 2560, 3840,
              4096, 4100, 7680, 32768] + [int(x) for x in rng.integers(1, 32769, size=60)]
    for w in widths:
        for base_align in (2, 4, 8, 16, 256):
            for extra in (0, 1, 3):
                stride = w + extra
                ref = 0x100000 + base_align
                cb, ng = api.load_shape(ref, ref + 0x4000000, w, stride, stride * 9, 2)
                assert (cb, ng) in LAUNCHED, (w, base_align, extra, cb, ng)
                align = 16
                for v in (ref, ref + 0x4000000, stride * 2, stride * 18):
                    while align > 1 and v % align:
                        align //= 2
                want_cb = next((c for c in (8, 4) if c <= align and w * 2 // c > 0), 0)
                assert cb == want_cb, (w, align, cb, want_cb)
                if cb:
                    nc = w * 2 // cb
                    nper = -(-nc // 64)
                    idles = {g: -(-nper // g) * g * 64 - nc for g in (15, 8, 5, 4)}
                    best = min(idles.values())
                    assert idles[ng] == best and ng == max(g for g in idles if idles[g] == best), \
                        (w, align, cb, ng, idles)
                else:
                    assert align < 4 or w * 2 < 4, (w, align)


# ------------------------------------------------ planted breaks (header) --

MUTANTS = {
    1: "a tie to the odd value in the one-term step",
    2: "the parity ignored",
    3: "the tree composed in reverse",
    4: "a run's units under the wrong binade",
    5: "the term-by-term fallback as exact adds",
    6: "no rounding at all",
    7: "a lane's run order reversed",
    8: "the closed form's +2 from an odd start forgotten",
    9: "a noise row's ties rounded to odd",
    10: "a crossing row's terms across the edge added as one exact sum",
    11: "a crossing row group's odd count taken from the row's first group",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_header_break_is_caught(tmp_path, mutant):
    """Each break planted in the step header makes the host emulation
    disagree with the oracle on at least one frame: the breaks the pages
    list for their header (ADR-1497, Consequences), a reversed run order, a
    closed form without its +2, noise ties to odd, and two breaks of the
    group step of a crossing row."""
    from bit_exact_frame_amd import build as b
    so = b.build_host_emu(os.path.join(tmp_path, f"libemu_m{mutant}.so"), mutant)
    lib = ctypes.CDLL(so)
    lib.bef_host_plane_units.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_ssize_t, ctypes.c_int, ctypes.c_uint,
                                         ctypes.POINTER(ctypes.c_uint64)]
    wrong = []
    for flags in (0, 32, 2):
        for name, p in planes():
            h, w = p.shape
            out = (ctypes.c_uint64 * 3)()
            assert lib.bef_host_plane_units(p.ctypes.data, w, h, w, 16, flags, out) == 0
            if out[2] != oracle_units(name)[1]:
                wrong.append((flags, name))
        if wrong:
            break
    if not wrong:  # the fast path's decisions, then the fast noise
        lib.bef_host_fast_units.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_ssize_t, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_uint64)]
        lib.bef_host_fast_noise.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_ssize_t, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_uint64)]
        for name, p in planes():
            h, w = p.shape
            out = (ctypes.c_uint64 * 3)()
            assert lib.bef_host_fast_units(p.ctypes.data, w, h, w, 16, out) == 0
            if out[0] == 1 and out[1] != oracle_units(name)[1]:
                wrong.append(("fast", name))
        o = oracle.Oracle()
        for name, r, d in noise_pairs():
            h, w = r.shape
            out = (ctypes.c_uint64 * 3)()
            assert lib.bef_host_fast_noise(r.ctypes.data, d.ctypes.data, w, h, w, 16, out) == 0
            v = np.array([out[1]], np.uint64).view(np.float64)[0]
            if out[0] == 1 and v != math.ldexp(o.psnr_sum(r, d, 16), 16):
                wrong.append(("fast noise", name))
    assert wrong, f"break '{MUTANTS[mutant]}' was not caught"


# ------------------------------------------------------------- C header --

C_CALLER = r"""
#include "bef.h"
/* Every entry point called with arguments of the declared types: the header
   is plain C99 and its declarations are what a C caller links against. */
int use_all(const void *r, const void *d, void *st, double *dres, uint64_t *u,
            uint8_t *paths, uint32_t *ceil_out) {
  double m[4], p[2], mom[8], ps[4], planes[1][7];
  const void *rs[1] = {r}, *ds[1] = {d};
  int ws[1] = {4}, hs[1] = {2};
  ptrdiff_t strides[1] = {4}, pitches[1] = {8};
  double ms = 0.0;
  long n = 0;
  int rc = moment_frame(r, d, 4, 2, 4, 10, m);
  rc |= psnr_noise(r, d, 4, 2, 4, 10, p);
  rc |= bef_frames(r, d, 4, 2, 4, 8, 2, 10, st, mom, ps);
  rc |= bef_frames_async(r, d, 4, 2, 4, 8, 2, 10, st, dres);
  rc |= bef_frames_noalloc(r, d, 4, 2, 4, 8, 2, 10, st, dres);
  rc |= bef_pipe_submit(r, d, 4, 2, 4, 8, 2, 10, st, dres);
  rc |= bef_pipe_join(0, st);
  rc |= bef_pipe_set_walk_cus(0);
  rc |= bef_planes(rs, ds, ws, hs, strides, pitches, 1, 1, 10, st, &planes[0][0]);
  rc |= bef_frames_host(r, d, 4, 2, 4, 8, 2, 10, 0, mom, ps);
  rc |= bef_frames_units(r, d, 4, 2, 4, 8, 2, 10, st, u);
  rc |= bef_walk_paths(paths, 6);
  rc |= bef_read_ceiling(r, d, 4, 2, 4, 8, 2, st, ceil_out);
  rc |= bef_timing_enable(0);
  rc |= bef_timing_read(0, &ms, &n);
  bef_timing_reset();
  (void)bef_debug_set(BEF_DBG_PLAN_WRONG | BEF_DBG_PLAN_NONE | BEF_DBG_TERMS_ONLY |
                      BEF_DBG_FORCE_ROUND | BEF_DBG_NO_STRETCH | BEF_DBG_NO_CLOSED_FORM |
                      BEF_DBG_SPLIT_LAUNCH);
  bef_release();
  return rc | (bef_last_error()[0] != 0);
}
"""


def test_header_is_c99_and_every_entry_point_links(tmp_path):
    """include/bef.h compiles as strict C99 (no C++ in the ABI), a C caller
    of every declared entry point with the declared argument types compiles
    without a warning, and links against libbef.so (no call is made: that
    needs a GPU)."""
    import shutil
    import subprocess
    from bit_exact_frame_amd import api
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = tmp_path / "use_all.c"
    src.write_text(C_CALLER)
    obj = tmp_path / "use_all.o"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-c",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(obj)],
                   check=True, capture_output=True, text=True)
    so = tmp_path / "libuse.so"
    # link as a shared object against libbef.so: every referenced symbol must
    # resolve there (the HIP runtime libbef.so itself needs may stay unresolved)
    subprocess.run([gcc, "-shared", "-o", str(so), str(obj), api.LIB_PATH,
                    "-Wl,--no-undefined", "-Wl,--allow-shlib-undefined"],
                   check=True, capture_output=True, text=True)
    names = set(re.findall(r"\b(bef_[a-z_]+|moment_frame|psnr_noise)\s*\(", C_CALLER))
    assert names >= set(declared(HEADER)) - {"defined"}, set(declared(HEADER)) - names
