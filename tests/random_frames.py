"""Seeded random frames whose second-moment sum crosses 2^53 or 2^54 at a
random row and column (tests only).

Each case is one ref plane of random width, stride padding and bit depth,
filled in raster order to an exact target a little below or above 2^53 (one
case in four: 2^54) with ``boundary._fill_to``, then a tail of one of three
kinds:
  - zeros (the sum ends at the target);
  - small codewords, whose float squares are odd below 4096 and tie once
    the sum is past 2^53 (ADR-1497, Context: the CPU's running sum rounds
    at every add past 2^53);
  - full-range samples, which carry the sum further.
The dis plane is zeros (the noise then crosses with the moment), full range
(a noise sum below 2^53) or ref with its lowest bit flipped at random (a
tiny noise sum).
"""
from __future__ import annotations

import functools

import numpy as np

import boundary
from checkers import t_table

TWO53 = 1 << 53
TWO54 = 1 << 54
N_CASES = 16      # through the host emulation (CPU) and on the GPU
N_GPU_CASES = 64  # on the GPU only (cases 16 and up are GPU-only)


@functools.lru_cache(maxsize=4)  # a few cases, not all of them, held at once
def case(k: int):
    """(ref[h, stride], dis[h, stride], w, bpc, label) of case k."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0xBEF, 4242, k])))
    w = int(rng.integers(512, 6001))
    stride = w + int(rng.choice([0, 0, 7, 8, 64]))
    bpc = int(rng.integers(9, 17))
    edge = TWO54 if k % 4 == 3 else TWO53
    target = edge + int(rng.integers(-(1 << 31), 1 << 31))
    lo = int(rng.choice([30000, 45000]))
    mean_t = float(t_table()[lo:].astype(np.float64).mean())
    tail_rows = int(rng.integers(1, 121))
    h = -(-int(target / mean_t * 1.03 + 4096) // w) + tail_rows
    flat = np.zeros(h * w, np.uint16)
    pos = boundary._fill_to(flat, 0, target, lo, 65536, rng, False)
    tail = k % 3
    if tail == 1:
        flat[pos:] = rng.integers(0, 4096, size=flat.size - pos)
    elif tail == 2:
        flat[pos:] = rng.integers(0, 65536, size=flat.size - pos)
    ref = np.full((h, stride), 0xFFFF, np.uint16)
    ref[:, :w] = flat.reshape(h, w)
    dis = np.full_like(ref, 0xFFFF)
    mode = k % 5
    if mode in (0, 3):
        dis[:, :w] = 0
    elif mode in (1, 4):
        dis[:, :w] = rng.integers(0, 65536, size=(h, w))
    else:
        dis[:, :w] = ref[:, :w] ^ rng.integers(0, 2, size=(h, w)).astype(np.uint16)
    label = (f"case {k}: {w}x{h} stride {stride} bpc {bpc}, target 2^{edge.bit_length() - 1}"
             f"{target - edge:+d} at sample {pos}, tail {('zeros', 'small', 'full')[tail]}, "
             f"dis {('zeros', 'full', 'ref^1', 'zeros', 'full')[mode]}")
    return ref, dis, w, bpc, label
