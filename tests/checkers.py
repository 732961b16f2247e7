"""Independent integer checkers for the oracle (tests only).

These re-derive the CPU loops' results from the IEEE-754 definition of
round-to-nearest-even on exact integers, with Python integers, and never call
the oracle or the HIP library.  Everything is counted in *units*: for a
scaler s = 2^k a float square of x/s is T(x) / s^2 with T(x) an integer, so
each step of the CPU's double loop is an integer operation (ADR-1497,
Decision: every step in units is the exact integer sum rounded to 53
significant bits, ties to even).
"""
from __future__ import annotations

import functools

import numpy as np

TWO53 = 1 << 53


def rne(n: int, bits: int) -> int:
    """Round the non-negative integer ``n`` to ``bits`` significant bits,
    ties to even (the IEEE binary rounding of an exact integer)."""
    if n < 0:
        raise ValueError("non-negative only")
    nb = n.bit_length()
    if nb <= bits:
        return n
    sh = nb - bits
    q = n >> sh
    r = n & ((1 << sh) - 1)
    half = 1 << (sh - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return q << sh


def rne53_add(s: int, t: int) -> int:
    """One step of the CPU's double accumulation, in units."""
    return rne(s + t, 53)


@functools.lru_cache(maxsize=None)
def t_table() -> np.ndarray:
    """T(x) = RNE24(x^2) for every 16-bit x, as uint64: the float32 square
    of x / s in units of 1/s^2 (exact for every s = 2^k)."""
    return np.array([rne(x * x, 24) for x in range(65536)], dtype=np.uint64)


def terms_moment(plane: np.ndarray) -> np.ndarray:
    """Raster-order second-moment terms (uint64) of an (h, w) plane."""
    return t_table()[plane.astype(np.int64).ravel()]


def terms_noise(ref: np.ndarray, dis: np.ndarray) -> np.ndarray:
    """(h, w) uint64 noise terms T(|r - d|)."""
    d = np.abs(ref.astype(np.int64) - dis.astype(np.int64))
    return t_table()[d]


def fold_rne53(terms) -> int:
    """The CPU's sequential double accumulation of non-negative integer
    ``terms``, in units, starting from 0.  The prefix that stays at or below
    2^53 is exact (every integer there is a double), so it is taken in bulk
    from an exact integer cumulative sum; the rest is folded one rounded
    step at a time (the body of ``rne`` at 53 bits, inlined for speed)."""
    t = np.asarray(terms, dtype=np.uint64)
    if t.size == 0:
        return 0
    cs = np.cumsum(t, dtype=np.uint64)  # exact: totals here stay < 2^64
    k = int(np.searchsorted(cs, np.uint64(TWO53), side="right"))
    s = int(cs[k - 1]) if k > 0 else 0
    for v in t[k:].tolist():
        n = s + v
        if n > TWO53:
            sh = n.bit_length() - 53
            r = n & ((1 << sh) - 1)
            if r:
                half = 1 << (sh - 1)
                n -= r
                if r > half or (r == half and (n >> sh) & 1):
                    n += 1 << sh
        s = n
    return s


def moment_units(plane: np.ndarray):
    """(S1, S2_cpu, S2_exact) in units for an (h, w) plane."""
    x = plane.astype(np.int64)
    s1 = int(x.sum())
    terms = terms_moment(plane)
    return s1, fold_rne53(terms), int(terms.sum(dtype=np.uint64))


def psnr_units(ref: np.ndarray, dis: np.ndarray):
    """(D_cpu, D_exact) in units: exact row sums, then the rows folded in
    order with rounding (ADR-1499, Decision, argument steps 1-3)."""
    rows = terms_noise(ref, dis).sum(axis=1, dtype=np.uint64)
    return fold_rne53(rows), int(rows.sum(dtype=np.uint64))
