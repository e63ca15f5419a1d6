"""GPU parity of the FP4 design-space variants (E2M1 with a block of 16 or
32 and an E4M3, E8M0 or BF16 block scale; "FP4 All the Way" summary,
Outline) against the oracle: codes, block scales and tensor exponents
bit-exact under nearest and stochastic rounding, row-wise and column-wise,
statistics within 1e-5, on shapes with ragged work tails and the method's
edge cases."""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from parity import compare_codes, compare_stats, gpu_codes, oracle_quant, say

pytestmark = pytest.mark.gpu

VARIANTS = [S.FP4_E4M3_B32, S.FP4_E8M0_B16, S.FP4_BF16_B16, S.FP4_BF16_B32]


def run(x, layout, fmt, rnd, seed=0, tid=0, amax=None):
    say(f"fp4 variant case layout={layout} fmt={fmt} rnd={rnd} shape={tuple(x.shape)} seed={seed}")
    amax_d = None if amax is None else torch.tensor([amax], dtype=torch.float32, device="cuda")
    q, st = S.quantize(x.cuda(), layout, fmt, rnd, seed, tid, amax=amax_d)
    torch.cuda.synchronize()
    o = oracle_quant(x, layout, fmt, rnd, seed, tid, amax=amax)
    what = f"layout={layout} fmt={fmt} rnd={rnd} shape={tuple(x.shape)}"
    compare_codes(gpu_codes(q), o, fmt, what=what)
    compare_stats(S.decode_stats(st)[0], o["stats"], what=what, check_err=o["stats"]["n_nonfinite"] == 0)
    return o


@pytest.mark.parametrize("fmt", VARIANTS)
@pytest.mark.parametrize("rnd", [S.RNE, S.SR])
def test_variant_parity(fmt, rnd):
    shapes = [(64, 64), (200, 96), (3, 4096), (544, 288)]
    for i, shp in enumerate(shapes):
        x = synth.gen_matrix(shp, seed=60 + i, std=1.0 if i % 2 else 2e-3)
        run(x, S.ROWWISE, fmt, rnd, seed=3, tid=7)
        if shp[0] % 32 == 0:
            run(x, S.COLWISE, fmt, rnd, seed=5, tid=9)


@pytest.mark.parametrize("fmt", VARIANTS)
def test_variant_edge_cases(fmt):
    z = torch.zeros((32, 64), dtype=torch.bfloat16)
    z[::2, 1::3] = -0.0
    o = run(z, S.ROWWISE, fmt, S.RNE)
    assert o["stats"]["sum_x2"] == 0.0
    run(torch.full((32, 64), 0.375, dtype=torch.bfloat16), S.COLWISE, fmt, S.SR, seed=9)
    for dist in ("lognormal_mixed", "student_t"):
        x = synth.gen_matrix((96, 256), seed=31, dist=dist)
        run(x, S.ROWWISE, fmt, S.SR, seed=1, tid=2)
        run(x, S.COLWISE, fmt, S.RNE, seed=1, tid=3)
    x = synth.gen_matrix((64, 128), seed=5)
    x[3, 17] = float("nan")
    x[40, 100] = float("inf")
    o = run(x, S.ROWWISE, fmt, S.RNE)
    assert o["stats"]["n_nonfinite"] == 2
    if fmt == S.FP4_E4M3_B32:                   # delayed scaling: a stale, smaller max saturates
        run(synth.gen_x(synth.WORKLOADS["linear512"], 0), S.ROWWISE, fmt, S.SR, seed=4, amax=8.0)


def test_variant_sizes_match_workload_tensors():
    """The tinyllama Gate layer's dY (4096 x 5632) in every variant, row-wise
    SR: sampled rows of the full-size result against the oracle."""
    wl = synth.WORKLOADS["tinyllama1b"]
    li = [l.name for l in wl.layers].index("Gate")
    dy = synth.gen_dy(wl, li)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(dy.shape[0], 48, replace=False), [0, dy.shape[0] - 1]]))
    for fmt in VARIANTS:
        say(f"fp4 variant full size fmt={fmt} shape={tuple(dy.shape)}")
        q, _ = S.quantize(dy.cuda(), S.ROWWISE, fmt, S.SR, 0, 2, with_stats=False)
        torch.cuda.synchronize()
        o = oracle_quant(dy, S.ROWWISE, fmt, S.SR, 0, 2, rows=rows)
        compare_codes(gpu_codes(q), o, fmt, rows=rows, what=f"full size fmt={fmt}")
