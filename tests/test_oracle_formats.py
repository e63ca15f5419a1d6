"""Pins for the oracle's number formats and rounding rules.

What pins what:
  * E2M1 value set: the closed set {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}.
  * E2M1 round-to-nearest: exhaustive over every finite bf16 magnitude against
    a brute-force nearest search written here (distance to all 8 values,
    ties to the even code), plus hand-worked tie points.
  * E4M3 decode/encode: torch's float8_e4m3fn (an independent library
    implementation) on every bf16 magnitude <= 448; saturation by hand.
  * Stochastic rounding: the expectation over all 2^16 draws must sit within
    one 2^-16 step below the input [Research on Mixed-Precision Training for
    LLMs, Core Techniques: stochastic rounding keeps the expected value].
"""
import numpy as np
import pytest
import torch

from oracle import formats as F

pytestmark = []


def all_bf16_magnitudes():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)     # +0 .. largest finite
    return (bits << 16).view(np.float32)


def test_e2m1_value_set():
    vals = F.e2m1_decode(np.arange(16))
    expect = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    assert set(np.abs(vals).tolist()) == expect
    assert sorted(vals[:8].tolist()) == sorted(expect)
    assert all(v <= 0 for v in vals[8:])
    assert np.signbit(vals[8])                        # code 0x8 is -0
    for c in range(16):
        v = np.float32(vals[c])
        assert F.e2m1_encode(np.array([v]), "rne")[0] == c
        assert F.e2m1_encode(np.array([v]), "sr", np.array([0xFFFF]))[0] == c


def brute_nearest(a, grid):
    d = np.abs(a[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    n = cand.sum(axis=1)
    first = np.argmax(cand, axis=1)
    even = np.where(cand[:, ::2].any(axis=1),
                    2 * np.argmax(cand[:, ::2], axis=1), first)
    return np.where(n > 1, even, first)


def test_e2m1_rne_exhaustive_bf16():
    for scale in (1.0, 2.0 ** -3, 2.0 ** 5, 1.0 / 3.0):
        with np.errstate(over="ignore"):
            a = (all_bf16_magnitudes() * np.float32(scale)).astype(np.float32)
        a = a[np.isfinite(a)]
        got = F.e2m1_encode(a, "rne").astype(np.int64)
        want = brute_nearest(np.minimum(a.astype(np.float64), 6.0), F.E2M1_GRID)
        assert np.array_equal(got, want)
        neg = F.e2m1_encode(-a, "rne").astype(np.int64)
        assert np.array_equal(neg, want | 8)


@pytest.mark.parametrize("a,idx", [
    (0.25, 0), (0.2500001, 1), (0.75, 2), (0.7499999, 1), (1.25, 2), (1.2500001, 3),
    (1.75, 4), (2.5, 4), (2.5000002, 5), (3.5, 6), (3.4999998, 5), (5.0, 6),
    (5.0000005, 7), (6.0, 7), (7.0, 7), (1e30, 7), (0.0, 0)])
def test_e2m1_rne_ties_hand(a, idx):
    assert F.e2m1_encode(np.array([a], np.float32), "rne")[0] == idx


def test_e4m3_decode_matches_torch():
    codes = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ok = np.isfinite(tv)
    assert ok.sum() == 254                            # 0x7F / 0xFF are NaN
    mine = F.e4m3_decode(np.arange(256)[ok])
    assert np.array_equal(mine, tv[ok])
    assert F.E4M3_GRID[0x7E] == 448.0 and F.E4M3_GRID[1] == 2.0 ** -9
    assert F.E4M3_GRID[8] == 2.0 ** -6


def test_e4m3_rne_matches_torch_exhaustive_bf16():
    a = all_bf16_magnitudes()
    for scale in (1.0, 1.0 / 3.0, 2.0 ** -7):
        v = (a * np.float32(scale)).astype(np.float32)
        v = v[v <= 448.0]
        v = np.concatenate([v, -v])
        got = F.e4m3_encode(v, "rne")
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, ref)


def test_e4m3_rne_random_fp32_matches_torch():
    rng = np.random.default_rng(5)
    v = np.exp2(rng.uniform(-14, 8.8, 200000)).astype(np.float32)
    v = v[v <= 448.0]
    got = F.e4m3_encode(v, "rne")
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("a,code", [
    (448.0, 0x7E), (463.99, 0x7E), (464.0, 0x7E), (1e9, 0x7E), (2.0 ** -9, 1),
    (2.0 ** -10, 0), (2.0 ** -10 * 1.0001, 1), (1.0625, 0x38), (1.1875, 0x3A),
    (1.5 * 2.0 ** -9, 2)])
def test_e4m3_rne_hand(a, code):
    assert F.e4m3_encode(np.array([a], np.float32), "rne")[0] == code


def sr_expectation(a, grid):
    """Mean of the decoded stochastic rounding of a over all 2^16 draws."""
    r16 = np.arange(65536)
    out = []
    for v in a:
        idx = F.stochastic_round(np.full(65536, v), grid, r16)
        out.append(grid[idx].mean())
    return np.array(out)


@pytest.mark.parametrize("grid_name", ["e2m1", "e4m3"])
def test_sr_expectation_over_all_draws(grid_name):
    grid = F.E2M1_GRID if grid_name == "e2m1" else F.E4M3_GRID
    rng = np.random.default_rng(11)
    top = grid[-1]
    a = rng.uniform(0, top, 300).astype(np.float32).astype(np.float64)
    a = np.concatenate([a, grid, (grid[:-1] + grid[1:]) / 2, [top * 0.999, 1e-30]])
    a = a.astype(np.float32).astype(np.float64)
    mean = sr_expectation(a, grid)
    lo = grid[np.clip(np.searchsorted(grid, a, side="right") - 1, 0, len(grid) - 2)]
    step = grid[np.clip(np.searchsorted(grid, a, side="right") - 1, 0, len(grid) - 2) + 1] - lo
    inside = a < top
    # unbiased to within one 2^-16 step, never above the input
    assert np.all(mean[inside] <= a[inside] + 1e-300)
    assert np.all(a[inside] - mean[inside] < step[inside] * 2.0 ** -16)
    # grid points are reproduced exactly; the top saturates
    on = np.isin(a, grid)
    assert np.all(mean[on] == a[on])


def test_sr_extreme_draws():
    grid = F.E2M1_GRID
    a = np.array([0.3, 1.2, 2.0, 2.0000002, 5.9999995], dtype=np.float32).astype(np.float64)
    lo = F.stochastic_round(a, grid, np.zeros(5, np.int64))
    hi = F.stochastic_round(a, grid, np.full(5, 65535))
    assert grid[lo].tolist() == [0.0, 1.0, 2.0, 2.0, 4.0]
    # r16 = 65535 rounds up iff frac >= 2^-16
    assert grid[hi].tolist() == [0.5, 1.5, 2.0, 2.0, 6.0]


def test_nibble_packing_order():
    codes = np.array([[1, 2, 3, 4, 0xF, 0]], np.uint8)
    packed = F.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(F.unpack_nibbles(packed), codes)
