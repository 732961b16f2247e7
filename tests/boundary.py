"""Seed-built 16-bit frames whose exact second-moment sum sits on 2^53 or
2^54 units (tests only).

The pages check their twins on four such frames: exact sums one unit below
2^53, exactly 2^53, 2^53 and then three ties the CPU drops, and 2^54 and
then seven unit terms it drops (ADR-1497, Decision; ADR-1499,
Consequences).  They do not say how those
frames were made; this builder is one reading: fill pixels in raster order
with seeded uniform samples while the remaining distance to the target is
large, then greedily place the largest sample whose float square (in units)
still fits, until the target is met exactly; zero the rest.  The exact sum is
asserted with Python integers.

The float square in units is T(x) = RNE24(x^2); the table comes from
``checkers`` (an integer re-derivation, pinned against the oracle's float32
square for all 65536 samples by the oracle tests).
"""
from __future__ import annotations

import numpy as np

from checkers import t_table

W, H = 3840, 2160
TWO53 = 1 << 53
TWO54 = 1 << 54


def _rng(tag: int):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0xBEF, 77, tag])))


def _fill_to(flat: np.ndarray, start: int, target: int, lo: int, hi: int,
             rng, even_only: bool) -> int:
    """Fill ``flat[start:]`` so that the exact T-sum of what is written equals
    ``target``; returns the index after the last written sample."""
    tt = t_table()
    n = flat.size
    cap = n - start
    # random part: stay at least 2^34 below the target
    draw = rng.integers(lo, hi, size=cap).astype(np.int64)
    if even_only:
        draw &= ~1
    cs = np.cumsum(tt[draw], dtype=np.uint64)
    k = int(np.searchsorted(cs, np.uint64(target - (1 << 34)), side="right"))
    if k >= cap:
        raise ValueError("frame too small for the target")
    flat[start:start + k] = draw[:k]
    rem = target - (int(cs[k - 1]) if k > 0 else 0)
    pos = start + k
    # greedy part: largest x with T(x) <= rem (T is non-decreasing in x)
    cand = np.arange(0, 65536, 2 if even_only else 1)
    tv = tt[cand].astype(object)
    tv_u = tt[cand]
    while rem > 0:
        j = int(np.searchsorted(tv_u, np.uint64(rem), side="right")) - 1
        if j <= 0:
            raise ValueError("greedy fill cannot meet the target")
        x = int(cand[j])
        flat[pos] = x
        pos += 1
        rem -= int(tv[j])
        if pos >= n:
            raise ValueError("frame too small for the greedy tail")
    return pos


def build(kind: str):
    """Return (plane[h, w] uint16, info dict) for one boundary frame kind:

    ``b53m1``  exact sum 2^53 - 1
    ``b53``    exact sum 2^53
    ``b53p3``  exact sum 2^53 over the first h-3 rows, then each of the last
               three rows holds one sample of value 1 (a tie each)
    ``odd53``  exact sum 2^53 - 2 over the first h-1 rows; the last row holds
               2, 100 and fifty 1s: the sum enters the binade of 2^53 with S/2
               odd and meets fifty ties there (a stretch from an odd start)
    ``b54p7``  exact sum 2^53, then only even samples (terms divisible by 4,
               so every add is exact in the binades of 2^53 and 2^54) up to
               exactly 2^54, then seven samples of value 1 at the end
    """
    plane = np.zeros((H, W), dtype=np.uint16)
    flat = plane.reshape(-1)
    body = (H - 3) * W
    if kind == "b53m1":
        _fill_to(flat[:body], 0, TWO53 - 1, 0, 65536, _rng(1), False)
    elif kind == "b53":
        _fill_to(flat[:body], 0, TWO53, 0, 65536, _rng(2), False)
    elif kind == "b53p3":
        _fill_to(flat[:body], 0, TWO53, 0, 65536, _rng(3), False)
        for r in (H - 3, H - 2, H - 1):
            plane[r, W // 2] = 1
    elif kind == "odd53":
        _fill_to(flat[:(H - 1) * W], 0, TWO53 - 2, 0, 65536, _rng(6), False)
        plane[H - 1, 0] = 2       # 2^53 - 2 + 4 = 2^53 + 2: S / 2 odd
        plane[H - 1, 1] = 100     # + 10000 exactly: still odd
        plane[H - 1, 2:52] = 1    # fifty ties from an odd start
    elif kind == "b54p7":
        pos = _fill_to(flat[:body], 0, TWO53, 32768, 65536, _rng(4), False)
        _fill_to(flat[:body], pos, TWO53, 32768, 65536, _rng(5), True)
        flat[flat.size - 7:] = 1
    else:
        raise KeyError(kind)
    return plane


KINDS = ("b53m1", "b53", "b53p3", "b54p7", "odd53")
