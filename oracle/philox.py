"""Philox4x32-10 counter-based generator and the per-element 16-bit draw.

The generator follows its published definition (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11): two 32x32->64-bit
multiplies per round with multipliers 0xD2511F53 and 0xCD9E8D57, Weyl key
increments 0x9E3779B9 and 0xBB67AE85, ten rounds.

Stochastic rounding of an element draws 16 uniform bits keyed on
(seed, tensor id, element index):
  key     = (seed mod 2^32, seed >> 32)
  counter = (g mod 2^32, g >> 32, tensor_id, 0),  g = idx >> 3
  word    = output word (idx >> 1) & 3
  R16     = (word >> (16 * (idx & 1))) & 0xFFFF
so one generator call serves eight consecutive elements. idx is the element
index in the quantized output layout (row * K + k).
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorised Philox4x32-10. Counters are arrays (or scalars) of uint32
    values; the key is two python ints. Returns four uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        p0 = M0 * c0            # < 2^64, exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


def r16(seed: int, tensor_id: int, idx: np.ndarray) -> np.ndarray:
    """16 random bits for each element index idx (uint64 array)."""
    idx = np.asarray(idx, dtype=np.uint64)
    g = idx >> np.uint64(3)
    w = philox4x32_10(g & MASK32, g >> np.uint64(32), np.uint64(tensor_id) + 0 * g,
                      0 * g, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    words = np.stack(w, axis=0)                       # [4, ...]
    sel = ((idx >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(words, sel[None, ...], axis=0)[0]
    shift = ((idx & np.uint64(1)) * np.uint64(16)).astype(np.uint32)
    return ((word >> shift) & np.uint32(0xFFFF)).astype(np.uint32)
