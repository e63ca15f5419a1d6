"""Stochastic rounding is unbiased on the GPU, at the full size of the 7B
Down-projection sweep (dY: T = 16384 x 4096, W^T: 11008 x 4096) with its ten
SR seeds ("Research on Mixed-Precision Training for LLMs", Core Techniques:
stochastic rounding keeps the expected value; "FP4 All the Way" summary,
Outline: SR in back-propagation).

For every element, the ten seeds give independent draws (one Philox stream
per seed), so with e_s = Q_s(x) - x:
  * sum_i mean_s(e_s(i)) / sqrt(sum_i var_s(i) / 10) is a standard normal
    statistic (elements are independent) and must lie within +-5;
  * mean_i mean_s(e_s(i))^2 must match mean_i var_s(i) / 10 within 5 %
    (the ten draws are independent: the variance of the mean shrinks
    tenfold).
Elements whose scaled value lies beyond the largest code are left out: they
saturate, deterministically (checked: every seed gives +-6 x block scale,
or +-448 for FP8). With the block scale rounded to nearest (NVFP4: E4M3 of
blockmax/6; MX-FP4: 2^(floor(log2 blockmax) - 2)) that is a few per cent of
the elements. The decoding of codes, scales and tensor exponents is done
here with the oracle's value tables.
"""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from oracle import formats as OF
from parity import say

pytestmark = pytest.mark.gpu

SEEDS = synth.WORKLOADS["down7b_sweep"].sr_seeds


def _tables(dev):
    e2m1 = torch.tensor(OF.E2M1_GRID, dtype=torch.float64, device=dev)
    e4m3 = torch.tensor(np.concatenate([OF.E4M3_GRID, [0.0]]), dtype=torch.float64, device=dev)
    return e2m1, e4m3


def dequant(q: S.QuantizedTensor):
    """fp64 values and the per-element largest representable magnitude."""
    dev = q.codes.device
    e2m1, e4m3 = _tables(dev)
    R, K = q.rows, q.k
    if q.format == S.FP8:
        c = q.codes.view(R, K).long()
        mag = e4m3[c & 0x7F]
        sign = torch.where((c & 0x80) != 0, -1.0, 1.0).double()
        t = 2.0 ** q.texp.item()
        return sign * mag * t, torch.full_like(mag, 448.0 * t)
    b = q.codes.view(R, K // 2).long()
    nib = torch.stack([b & 0xF, b >> 4], dim=-1).view(R, K)
    val = torch.where((nib & 8) != 0, -1.0, 1.0).double() * e2m1[nib & 7]
    if q.format == S.NVFP4:
        sc = e4m3[q.scales.view(R, K // 16).long()].repeat_interleave(16, dim=1)
        t = 2.0 ** q.texp.item()
        return val * sc * t, 6.0 * sc * t
    sc = torch.pow(2.0, q.scales.view(R, K // 32).double() - 127.0).repeat_interleave(32, dim=1)
    return val * sc, 6.0 * sc


def unbiased_check(x: torch.Tensor, layout: int, fmt: int, tensor_id: int, what: str):
    say(f"SR unbiasedness {what} fmt={fmt} layout={layout} seeds={len(SEEDS)} shape={tuple(x.shape)}")
    ref = x.double() if layout == S.ROWWISE else x.t().double()
    s1 = torch.zeros_like(ref)
    s2 = torch.zeros_like(ref)
    keep = None
    for seed in SEEDS:
        q, _ = S.quantize(x, layout, fmt, S.SR, seed, tensor_id, with_stats=False)
        v, lim = dequant(q)
        e = v - ref
        s1 += e
        s2 += e * e
        k = ref.abs() <= lim
        sat = ~k
        assert torch.equal(v[sat], torch.sign(ref[sat]) * lim[sat]), f"{what}: saturation not exact"
        keep = k if keep is None else keep & k
        del q, v, lim, e
    n = float(len(SEEDS))
    mean = s1 / n
    var = (s2 - n * mean * mean) / (n - 1.0)
    m, v = mean[keep], var[keep]
    z = m.sum().item() / np.sqrt(v.sum().item() / n)
    ratio = (m * m).mean().item() / (v.mean().item() / n)
    frac = keep.double().mean().item()
    say(f"  kept {frac:.6f} of elements; z = {z:+.3f}; variance-of-mean ratio = {ratio:.4f}")
    assert frac > 0.95
    assert abs(z) < 5.0, f"{what}: SR mean error z = {z}"
    assert abs(ratio - 1.0) < 0.05, f"{what}: variance of the seed mean off by {ratio}"


@pytest.mark.parametrize("fmt", [S.NVFP4, S.FP8, S.MXFP4])
def test_sr_unbiased_dy_rowwise(fmt):
    wl = synth.WORKLOADS["down7b_sweep"]
    dy = synth.gen_dy(wl, 0).cuda()
    unbiased_check(dy, S.ROWWISE, fmt, 2, "dY row-wise")
    del dy
    torch.cuda.empty_cache()


def test_sr_unbiased_w_colwise_nvfp4():
    wl = synth.WORKLOADS["down7b_sweep"]
    w = synth.gen_w(wl, 0).cuda()
    unbiased_check(w, S.COLWISE, S.NVFP4, 3, "W column-wise")
    del w
    torch.cuda.empty_cache()
