"""Pins for the oracle's quantizers and statistics.

  * tensor exponent: closed-form window of max|x| / 2^eS;
  * NVFP4 / FP8 / MX round trips: tensors built from representable values
    (code x block scale x tensor scale) must reproduce codes, scales and the
    tensor exactly under both roundings, with zero squared error;
  * round-to-nearest error is at most half a grid step of the scaled value;
  * stochastic rounding through the whole quantizer is unbiased over many
    seeds [Research on Mixed-Precision Training for LLMs, Core Techniques];
  * MX scale: the OCP rule puts each block max in [4, 8) after scaling;
  * statistics: closed forms on constant tensors, exact zero error on
    representable tensors, non-finite counting;
  * row subsets (used for sampled parity at full size) agree with the whole.
"""
import numpy as np
import pytest

from oracle import formats as F
from oracle import quantize as Q

NVFP4, FP8, MXFP4, BF16 = Q.NVFP4, Q.FP8, Q.MXFP4, Q.BF16


def bf16_round(a):
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("amax", [1.0, 2688.0, 2688.0001, 1344.0, 1e-3, 3.0e38, 7.1e-39, 71.0, 1.3125 * 2 ** 11])
def test_nvfp4_tensor_exp_window(amax):
    a = float(np.float32(amax))
    e = Q.pow2_tensor_exp(a, 6 * 448)
    assert 1344.0 < a * 2.0 ** -e <= 2688.0
    e8 = Q.pow2_tensor_exp(a, 448)
    assert 224.0 < a * 2.0 ** -e8 <= 448.0
    assert Q.pow2_tensor_exp(0.0, 448) == 0


def _representable_nvfp4(R, nb, rng, eS):
    """Blocks of E2M1 codes with one +-6 per block, random E4M3 scales with the
    largest in (224, 448] so the tensor exponent is eS."""
    codes = rng.integers(0, 16, size=(R, nb, 16)).astype(np.uint8)
    pos = rng.integers(0, 16, size=(R, nb))
    np.put_along_axis(codes, pos[:, :, None], (7 | (rng.integers(0, 2, (R, nb, 1)) << 3)).astype(np.uint8), axis=2)
    sc = rng.integers(8, 0x7E, size=(R, nb)).astype(np.uint8)    # normal E4M3 scales
    sc[0, 0] = 0x7E                                               # 448 -> block max 2688
    x = F.e2m1_decode(codes) * F.e4m3_decode(sc)[:, :, None] * 2.0 ** eS
    return x.reshape(R, nb * 16).astype(np.float32), codes.reshape(R, nb * 16), sc


@pytest.mark.parametrize("eS", [-12, 0, 3])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_nvfp4_round_trip_exact(eS, rounding):
    rng = np.random.default_rng(100 + eS)
    x, codes, sc = _representable_nvfp4(6, 5, rng, eS)
    assert np.array_equal(bf16_round(x), x)                       # bf16-representable
    q = Q.quantize(x, NVFP4, rounding, seed=9, tensor_id=4)
    assert q["texp"] == eS
    assert np.array_equal(q["scales"], sc)
    mags = codes & 7
    got = q["codes"]
    # +-0 codes may differ only in sign of zero when the value is zero
    assert np.array_equal(got & 7, mags)
    nz = mags != 0
    assert np.array_equal(got[nz], codes[nz])
    assert np.array_equal(q["xhat"], x.astype(np.float64))
    assert q["stats"]["sum_err2"] == 0.0


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_fp8_round_trip_exact(rounding):
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7F, size=(8, 48)).astype(np.uint8) | (rng.integers(0, 2, (8, 48)) << 7).astype(np.uint8)
    codes[0, 0] = 0x7E                                            # 448
    x = (F.e4m3_decode(codes) * 2.0 ** -5).astype(np.float32)
    q = Q.quantize(x, FP8, rounding, seed=1, tensor_id=3)
    assert q["texp"] == -5
    assert np.array_equal(q["xhat"], x.astype(np.float64))
    nz = (codes & 0x7F) != 0
    assert np.array_equal(q["codes"][nz], codes[nz])


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_mx_round_trip_exact(rounding):
    rng = np.random.default_rng(2)
    R, nb = 4, 6
    codes = rng.integers(0, 16, size=(R, nb, 32)).astype(np.uint8)
    codes[:, :, 0] = 7                                            # block max 6 -> X = exponent
    X = rng.integers(-20, 20, size=(R, nb))
    x = (F.e2m1_decode(codes) * np.exp2(X)[:, :, None]).reshape(R, nb * 32).astype(np.float32)
    q = Q.quantize(x, MXFP4, rounding, seed=5, tensor_id=1)
    assert np.array_equal(q["scales"].astype(np.int64) - 127, X)
    assert np.array_equal(q["xhat"], x.astype(np.float64))


def test_mx_scale_rule():
    rng = np.random.default_rng(4)
    x = bf16_round(rng.standard_normal((16, 256)) * np.exp2(rng.uniform(-10, 10, (16, 1))))
    q = Q.quantize(x, MXFP4, "rne")
    a_b = np.abs(x.reshape(16, 8, 32)).max(axis=2).astype(np.float64)
    X = q["scales"].astype(np.int64) - 127
    ratio = a_b / np.exp2(X)
    assert np.all((ratio >= 4.0) & (ratio < 8.0))


@pytest.mark.parametrize("fmt", [NVFP4, MXFP4, FP8])
def test_rne_error_at_most_half_step(fmt):
    rng = np.random.default_rng(7)
    x = bf16_round(rng.standard_normal((32, 128)) * 0.37)
    q = Q.quantize(x, fmt, "rne")
    xhat = q["xhat"]
    if fmt == NVFP4:
        s = np.repeat(F.e4m3_decode(q["scales"]), 16, axis=1) * 2.0 ** q["texp"]
        grid = F.E2M1_GRID
    elif fmt == MXFP4:
        s = np.repeat(np.exp2(q["scales"].astype(np.int64) - 127.0), 32, axis=1)
        grid = F.E2M1_GRID
    else:
        s = np.full(x.shape, 2.0 ** q["texp"])
        grid = F.E4M3_GRID
    r = np.abs(x.astype(np.float64)) / s
    qa = np.abs(xhat) / s
    # half of the larger neighbouring step, plus the fp32 rounding of r
    gi = np.clip(np.searchsorted(grid, qa), 0, len(grid) - 1)
    step_hi = grid[np.minimum(gi + 1, len(grid) - 1)] - grid[gi]
    step_lo = grid[gi] - grid[np.maximum(gi - 1, 0)]
    half = 0.5 * np.maximum(step_hi, step_lo)
    sat = r > grid[-1]
    assert np.all((np.abs(r - qa) <= half * (1 + 1e-6)) | (sat & (qa == grid[-1])))


def test_sr_unbiased_over_seeds():
    rng = np.random.default_rng(8)
    x = bf16_round(rng.standard_normal((4, 64)))
    n_seeds = 1000
    acc = np.zeros(x.shape)
    for s in range(n_seeds):
        acc += Q.quantize(x, NVFP4, "sr", seed=s, tensor_id=2)["xhat"]
    mean = acc / n_seeds
    q0 = Q.quantize(x, NVFP4, "rne")
    s_val = np.repeat(F.e4m3_decode(q0["scales"]), 16, axis=1) * 2.0 ** q0["texp"]
    r = np.abs(x) / s_val
    gi = np.clip(np.searchsorted(F.E2M1_GRID, r, side="right") - 1, 0, 6)
    step = (F.E2M1_GRID[gi + 1] - F.E2M1_GRID[gi]) * s_val
    p = np.clip((r - F.E2M1_GRID[gi]) * s_val / step, 0, 1)
    sd = np.sqrt(p * (1 - p) / n_seeds) * step
    dev = np.abs(mean - x)
    # the block max can exceed 6 x scale when the E4M3 scale rounds down:
    # those elements saturate deterministically to +-6 x scale
    sat = r > 6.0
    assert sat.sum() < 0.1 * x.size
    assert np.array_equal(mean[sat], np.sign(x[sat]) * 6.0 * s_val[sat])
    ok = ~sat
    assert np.all(dev[ok] <= 5 * sd[ok] + step[ok] * 2.0 ** -16 + 1e-12)
    # aggregate z-test over the unsaturated elements
    z = np.sum((mean - x)[ok]) / np.sqrt(np.sum(sd[ok] ** 2))
    assert abs(z) < 5


def test_stats_closed_forms():
    x = np.full((4, 32), 0.75, np.float32)
    for fmt in (NVFP4, FP8, MXFP4, BF16):
        q = Q.quantize(x, fmt, "rne")
        assert q["stats"]["sum_x2"] == 4 * 32 * 0.5625
        assert q["stats"]["amax"] == 0.75
        assert q["stats"]["sum_err2"] == 0.0            # constant blocks are exact
    x2 = x.copy()
    x2[1, 3] = np.nan
    x2[2, 5] = np.inf
    q = Q.quantize(x2, NVFP4, "rne")
    assert q["stats"]["n_nonfinite"] == 2
    assert q["stats"]["amax"] == 0.75
    assert q["bad_blocks"].sum() == 32                   # two 16-blocks


def test_signed_zero_codes():
    x = np.zeros((1, 32), np.float32)
    x[0, 1::2] = -0.0
    q = Q.quantize(x, NVFP4, "rne")
    assert q["codes"][0, 0::2].tolist() == [0] * 16
    assert q["codes"][0, 1::2].tolist() == [8] * 16
    assert q["scales"].tolist() == [[0, 0]]


@pytest.mark.parametrize("fmt", [NVFP4, FP8, MXFP4])
def test_row_subset_matches_full(fmt):
    rng = np.random.default_rng(10)
    x = bf16_round(rng.standard_normal((64, 64)))
    full = Q.quantize(x, fmt, "sr", seed=3, tensor_id=11)
    rows = np.array([0, 7, 63, 20])
    sub = Q.quantize(x[rows], fmt, "sr", seed=3, tensor_id=11, amax=Q.tensor_amax(x), row_ids=rows)
    assert np.array_equal(sub["codes"], full["codes"][rows])
    if fmt != FP8:
        assert np.array_equal(sub["scales"], full["scales"][rows])
    colw = Q.quantize_colwise(x, fmt, "sr", seed=3, tensor_id=11)
    cols = np.array([5, 0, 63])
    colsub = Q.quantize_colwise(x, fmt, "sr", seed=3, tensor_id=11, col_ids=cols)
    assert np.array_equal(colsub["codes"], colw["codes"][cols])


def test_supplied_max_sets_scale_stats_report_own_max():
    """Delayed scaling: a supplied max (8.0 = 1.0 * 2^3) fixes the tensor
    exponent by the closed forms (NVFP4 3 - 11 = -8, FP8 3 - 8 = -5), while
    the max|x| statistic stays the tensor's own (0.75); a constant block is
    still represented exactly (NVFP4: 0.75 * 2^8 = 192, block scale 32, code
    6; FP8: 0.75 * 2^5 = 24, an E4M3 value)."""
    x = np.full((4, 32), 0.75, np.float32)
    for fmt, e in ((NVFP4, -8), (FP8, -5)):
        q = Q.quantize(x, fmt, "rne", amax=8.0)
        assert q["texp"] == e
        assert q["stats"]["amax"] == 0.75
        assert q["stats"]["sum_err2"] == 0.0
        assert np.all(q["xhat"] == 0.75)
    # a smaller supplied max saturates: 0.75 with max 0.25 -> FP8 eS = -9 (0.25 = 2^-2),
    # 0.75 * 2^9 = 384 is still an E4M3 value; NVFP4 eS = -2 - 11 + 0 = -13 and the block
    # scale saturates at 448: 0.75 * 2^13 / 6 = 1024 -> 448, r = 6144 / 448 > 6 -> 6
    q = Q.quantize(x, NVFP4, "rne", amax=0.25)
    assert q["texp"] == -13
    assert np.all(q["xhat"] == 6.0 * 448.0 * 2.0 ** -13)
    assert q["stats"]["amax"] == 0.75
