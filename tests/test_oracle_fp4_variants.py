"""Pins for the FP4 design-space variants of the oracle (E2M1 codes with a
block of 16 or 32 and an E4M3, E8M0 or BF16 block scale; "FP4 All the Way"
summary, Outline: block size, scaling format and rounding were explored).

  * the BF16 scale encoder equals torch's float -> bfloat16 conversion
    (round to nearest even) on every positive fp32 pattern of a wide sample
    and on all ties;
  * each variant's block scale is what its rule gives from an independent
    codec: torch's float8_e4m3fn for E4M3, frexp for E8M0, torch's bfloat16
    for BF16 (a dropped term or a wrong block length fails here);
  * tensors built from representable values (code x block scale [x tensor
    scale]) round-trip exactly under both roundings;
  * nearest rounding errs by at most half a grid step; stochastic rounding
    is unbiased over many seeds [Research on Mixed-Precision Training for
    LLMs, Core Techniques];
  * the (16, E4M3) and (32, E8M0) rules give NVFP4 and MX-FP4 exactly.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quantize as Q

VARIANTS = [Q.FP4_E4M3_B32, Q.FP4_E8M0_B16, Q.FP4_BF16_B16, Q.FP4_BF16_B32]


def bf16_round(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def test_bf16_scale_encoder_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 0x7F7F0000, size=400000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 0x7F7F, size=20000).astype(np.uint32) << 16) | np.uint32(0x8000)
    t = np.concatenate([bits, ties, np.array([0, 1, 0x8000, 0x18000, 0x7F7F7FFF], np.uint32)]).view(np.float32)
    mine = F.bf16_scale_encode(t)
    ref = torch.from_numpy(t.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(F.bf16_decode(mine), torch.from_numpy(mine.view(np.int16).copy())
                          .view(torch.bfloat16).double().numpy())


def _data(R=16, K=256, seed=3):
    rng = np.random.default_rng(seed)
    return bf16_round(rng.standard_normal((R, K)) * np.exp2(rng.uniform(-12, 6, (R, 1))))


@pytest.mark.parametrize("fmt", VARIANTS + [Q.NVFP4, Q.MXFP4])
def test_block_scale_rule(fmt):
    x = _data()
    blk, kind = Q.FP4_VARIANT[fmt]
    q = Q.quantize(x, fmt, "rne")
    R, K = x.shape
    if kind == "e4m3":
        eS = Q.pow2_tensor_exp(Q.tensor_amax(x), 6.0 * 448.0)
        a_b = np.abs(np.ldexp(x, -eS).reshape(R, K // blk, blk)).max(axis=2).astype(np.float32)
        t = torch.from_numpy((a_b / np.float32(6.0)).astype(np.float32))
        ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert q["texp"] == eS
        assert np.array_equal(q["scales"], ref)
    elif kind == "e8m0":
        a_b = np.abs(x.reshape(R, K // blk, blk)).max(axis=2).astype(np.float64)
        X = np.frexp(a_b)[1] - 1 - 2
        assert np.array_equal(q["scales"].astype(np.int64) - 127, X)
    else:
        a_b = np.abs(x.reshape(R, K // blk, blk)).max(axis=2).astype(np.float32)
        ref = torch.from_numpy((a_b / np.float32(6.0)).astype(np.float32)).to(torch.bfloat16)
        assert np.array_equal(q["scales"], ref.view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("fmt", VARIANTS)
@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_round_trip_exact(fmt, rounding):
    rng = np.random.default_rng(5)
    blk, kind = Q.FP4_VARIANT[fmt]
    R, nb = 4, 6
    codes = rng.integers(0, 16, size=(R, nb, blk)).astype(np.uint8)
    codes[:, :, 0] = 7                                         # block max 6 x scale
    if kind == "e8m0":
        s = np.exp2(rng.integers(-20, 20, size=(R, nb)).astype(np.float64))
    elif kind == "e4m3":
        # E4M3 normal scales (t = 6 s / 6 exactly) and a power-of-two tensor scale
        sc = rng.integers(0x08, 0x7F, size=(R, nb))
        s = F.e4m3_decode(sc)
        s[0, 0] = 448.0                                        # the tensor max maps to 6 x 448
    else:
        s = bf16_round(np.exp2(rng.uniform(-30, 30, size=(R, nb)))).astype(np.float64)
    x = (F.e2m1_decode(codes) * s[:, :, None]).reshape(R, nb * blk)
    if kind == "e4m3":
        x = np.ldexp(x, -7)
    x = x.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), (F.e2m1_decode(codes) * s[:, :, None]).reshape(R, -1)
                          * (2.0 ** -7 if kind == "e4m3" else 1.0))
    q = Q.quantize(x, fmt, rounding, seed=5, tensor_id=1)
    assert np.array_equal(q["xhat"], x.astype(np.float64))
    assert q["stats"]["sum_err2"] == 0.0


def test_nvfp4_and_mx_are_variants():
    x = _data(seed=9)
    for fmt in (Q.NVFP4, Q.MXFP4):
        blk, kind = Q.FP4_VARIANT[fmt]
        twin = {("e4m3", 16): Q.NVFP4, ("e8m0", 32): Q.MXFP4}[(kind, blk)]
        assert twin == fmt
    # (32, E4M3) on blocks whose halves share the max equals NVFP4 per 16
    rng = np.random.default_rng(1)
    h = bf16_round(rng.standard_normal((8, 16)))
    x2 = np.repeat(h[:, None, :], 2, axis=1).reshape(8, 32)
    a = Q.quantize(x2, Q.FP4_E4M3_B32, "rne")
    b = Q.quantize(x2, Q.NVFP4, "rne")
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"][:, 0], b["scales"][:, 0])


@pytest.mark.parametrize("fmt", VARIANTS)
def test_rne_error_at_most_half_step(fmt):
    x = _data(32, 128, seed=7)
    blk, kind = Q.FP4_VARIANT[fmt]
    q = Q.quantize(x, fmt, "rne")
    if kind == "e4m3":
        s = np.repeat(F.e4m3_decode(q["scales"]), blk, axis=1) * 2.0 ** q["texp"]
    elif kind == "e8m0":
        s = np.repeat(np.exp2(q["scales"].astype(np.int64) - 127.0), blk, axis=1)
    else:
        s = np.repeat(F.bf16_decode(q["scales"]), blk, axis=1)
    grid = F.E2M1_GRID
    r = np.abs(x.astype(np.float64)) / s
    qa = np.abs(q["xhat"]) / s
    gi = np.clip(np.searchsorted(grid, qa), 0, len(grid) - 1)
    step_hi = grid[np.minimum(gi + 1, len(grid) - 1)] - grid[gi]
    step_lo = grid[gi] - grid[np.maximum(gi - 1, 0)]
    half = 0.5 * np.maximum(step_hi, step_lo)
    sat = r > grid[-1]
    assert np.all((np.abs(r - qa) <= half * (1 + 1e-6)) | (sat & (qa == grid[-1])))


@pytest.mark.parametrize("fmt", [Q.FP4_E8M0_B16, Q.FP4_BF16_B32])
def test_sr_unbiased_over_seeds(fmt):
    x = _data(4, 64, seed=8)
    n = 600
    acc = np.zeros(x.shape)
    for sd in range(n):
        acc += Q.quantize(x, fmt, "sr", seed=sd, tensor_id=4)["xhat"]
    mean = acc / n
    q0 = Q.quantize(x, fmt, "rne")
    blk, kind = Q.FP4_VARIANT[fmt]
    s = (np.repeat(np.exp2(q0["scales"].astype(np.int64) - 127.0), blk, axis=1) if kind == "e8m0"
         else np.repeat(F.bf16_decode(q0["scales"]), blk, axis=1))
    r = np.abs(x) / s
    sat = r > 6.0
    ok = ~sat
    gi = np.clip(np.searchsorted(F.E2M1_GRID, r, side="right") - 1, 0, 6)
    step = (F.E2M1_GRID[np.minimum(gi + 1, 7)] - F.E2M1_GRID[gi]) * s
    p = np.clip((r * s - F.E2M1_GRID[gi] * s) / np.where(step > 0, step, 1), 0, 1)
    sdv = np.sqrt(p * (1 - p) / n) * step
    z = np.sum((mean - x)[ok]) / np.sqrt(np.sum(sdv[ok] ** 2) + 1e-300)
    assert abs(z) < 5
    assert np.array_equal(mean[sat], np.sign(x[sat]) * 6.0 * s[sat])
