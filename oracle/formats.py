"""Number formats: E2M1 (FP4), E4M3 (FP8, OCP "fn" variant) and E8M0.

[FP4 All the Way summary, Outline]: the FP4 element format is E2M1 and the
shared 16-element block scale is stored in E4M3. The E2M1 magnitude set is
{0, 0.5, 1, 1.5, 2, 3, 4, 6}; E4M3 has bias 7, subnormals m * 2^-9 and a
largest finite value 448 (code 0x7E); 0x7F/0xFF are NaN and never produced.

Encoders here work from the value tables by nearest-value search; they do not
use bit tricks, so they can be read against the definitions directly.

Readings:
  * round-to-nearest breaks ties to the even code (IEEE default);
  * values beyond the largest finite magnitude saturate (E2M1 -> 6,
    E4M3 -> 448): the formats carry no infinities;
  * stochastic rounding: with lo <= |r| < hi the neighbouring grid points,
    frac = (|r| - lo) / (hi - lo); the magnitude rounds up iff
    R16 + floor(frac * 2^16) >= 2^16 for a uniform 16-bit R16, so
    P(up) = floor(frac * 2^16) / 2^16 (unbiased to within 2^-16 of a step).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- E2M1 (FP4)
# magnitude index 0..7 -> value; code = sign << 3 | index
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_GRID[codes & 7]
    return np.where(codes & 8, -mag, mag)


# ---------------------------------------------------------------- E4M3 (FP8)
def _e4m3_table() -> np.ndarray:
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_GRID = _e4m3_table()  # codes 0..126, strictly increasing; 0x7E = 448
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes).astype(np.int64)
    mag_code = codes & 0x7F
    if np.any(mag_code == 0x7F):
        raise ValueError("E4M3 NaN code")
    mag = E4M3_GRID[mag_code]
    return np.where(codes & 0x80, -mag, mag)


# ---------------------------------------------------------------- E8M0
def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes).astype(np.int64)
    if np.any(codes == 255):
        raise ValueError("E8M0 NaN code")
    return np.ldexp(1.0, codes - 127)


# ---------------------------------------------------------------- BF16 (as a block scale)
def bf16_scale_encode(t: np.ndarray) -> np.ndarray:
    """Round non-negative finite fp32 values to bfloat16, nearest with ties
    to the even code: the two bf16 neighbours are the fp32 pattern with its
    low 16 bits cleared and that plus one bf16 step; the nearer one wins, a
    tie goes to the one whose last kept bit is 0. Returns the 16-bit codes."""
    t = np.asarray(t, dtype=np.float32)
    bits = t.view(np.uint32).astype(np.uint64)
    lo = bits & np.uint64(0xFFFF0000)
    hi = lo + np.uint64(0x10000)
    rem = bits - lo                                    # distance above lo, in fp32 ulps
    half = np.uint64(0x8000)
    lo_even = (lo >> np.uint64(16)) & np.uint64(1) == 0
    up = (rem > half) | ((rem == half) & ~lo_even)
    return (np.where(up, hi, lo) >> np.uint64(16)).astype(np.uint16)


def bf16_decode(codes: np.ndarray) -> np.ndarray:
    return (np.asarray(codes, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- rounding
def round_nearest_even(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to a >= 0; ties go to the even index;
    values above the grid saturate to its last index."""
    a = np.asarray(a, dtype=np.float64)
    if np.any(a < 0) or np.any(np.isnan(a)):
        raise ValueError("magnitudes must be >= 0 and not NaN")
    n = len(grid)
    hi = np.searchsorted(grid, a, side="left")          # first grid >= a
    hi = np.minimum(hi, n - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= grid[-1], n - 1, idx)
    return idx.astype(np.int64)


def stochastic_round(a: np.ndarray, grid: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """Index of the stochastically rounded grid value for a >= 0.

    Let lo <= a < hi be the neighbouring grid values. The result is hi iff
    r16 + floor(frac * 65536) >= 65536, frac = (a - lo) / (hi - lo), else lo.
    Values at or above the last grid value give the last index.
    Every quantity is exact in fp64 (a is an fp32 value, grid steps are powers
    of two).
    """
    a = np.asarray(a, dtype=np.float64)
    r16 = np.asarray(r16).astype(np.int64)
    if np.any(a < 0) or np.any(np.isnan(a)):
        raise ValueError("magnitudes must be >= 0 and not NaN")
    n = len(grid)
    top = a >= grid[-1]
    lo = np.searchsorted(grid, a, side="right") - 1       # last grid <= a
    lo = np.clip(lo, 0, n - 2)
    step = grid[lo + 1] - grid[lo]
    frac = (a - grid[lo]) / step
    nfrac = np.floor(frac * 65536.0).astype(np.int64)
    up = (r16 + nfrac) >= 65536
    idx = np.where(up, lo + 1, lo)
    return np.where(top, n - 1, idx).astype(np.int64)


def e2m1_encode(r: np.ndarray, rounding: str, r16=None) -> np.ndarray:
    """fp32 values -> E2M1 codes (sign from the sign bit of r, so -0 -> 0x8)."""
    r = np.asarray(r, dtype=np.float32)
    a = np.abs(r).astype(np.float64)
    if rounding == "rne":
        idx = round_nearest_even(a, E2M1_GRID)
    elif rounding == "sr":
        idx = stochastic_round(a, E2M1_GRID, r16)
    else:
        raise ValueError(rounding)
    return (idx | (np.signbit(r).astype(np.int64) << 3)).astype(np.uint8)


def e4m3_encode(r: np.ndarray, rounding: str, r16=None) -> np.ndarray:
    """fp32 values -> E4M3 codes with saturation at 448."""
    r = np.asarray(r, dtype=np.float32)
    a = np.abs(r).astype(np.float64)
    if rounding == "rne":
        idx = round_nearest_even(a, E4M3_GRID)
    elif rounding == "sr":
        idx = stochastic_round(a, E4M3_GRID, r16)
    else:
        raise ValueError(rounding)
    return (idx | (np.signbit(r).astype(np.int64) << 7)).astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[R, K] 4-bit codes -> [R, K/2] bytes, element k in the low nibble when
    k is even."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out
