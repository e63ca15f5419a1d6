"""GPU parity: the block-scaled MFMA GEMMs against the oracle's fp64 product
of the dequantized operands, within 1e-5 * sum_k |a_k||b_k| per element.

The operands are quantized by the oracle and uploaded, so this isolates the
GEMM from the GPU quantizers; shapes span several 128x128 output tiles and
ragged M / N tails."""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from parity import check_gemm, oracle_quant, say, upload_oracle_q

pytestmark = pytest.mark.gpu

SHAPES = [(128, 128, 128), (200, 72, 256), (16, 16, 128), (384, 256, 512), (1, 1, 128),
          (257, 129, 384), (64, 520, 1024)]


def run(fmt, M, N, K, seed, dist="normal", rnd_b=S.SR):
    say(f"gemm case fmt={fmt} M={M} N={N} K={K} seed={seed} dist={dist}")
    a = synth.gen_matrix((M, K), seed=seed, dist=dist)
    b = synth.gen_matrix((N, K), seed=seed + 1000, std=0.02, dist=dist)
    oa = oracle_quant(a, S.ROWWISE, fmt, S.RNE, 0, 0)
    ob = oracle_quant(b, S.ROWWISE, fmt, rnd_b, 1, 1)
    qa, qb = upload_oracle_q(oa, fmt), upload_oracle_q(ob, fmt)
    c = S.qgemm(qa, qb)
    torch.cuda.synchronize()
    return check_gemm(c.cpu().numpy().astype(np.float64), oa["xhat"], ob["xhat"],
                      what=f"fmt={fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", [S.NVFP4, S.FP8, S.MXFP4, S.BF16])
def test_gemm_parity(fmt):
    for i, (M, N, K) in enumerate(SHAPES):
        run(fmt, M, N, K, seed=100 + i)


@pytest.mark.parametrize("fmt", [S.NVFP4, S.FP8, S.MXFP4])
def test_gemm_wide_range(fmt):
    run(fmt, 128, 96, 256, seed=7, dist="lognormal_mixed")
    run(fmt, 96, 128, 384, seed=8, dist="student_t")


def test_gemm_tensor_scale_epilogue():
    # tensors whose tensor exponents are far from 0 in both directions
    for fmt in (S.NVFP4, S.FP8):
        a = synth.gen_matrix((64, 256), seed=1, std=3e4)
        b = synth.gen_matrix((48, 256), seed=2, std=1e-6)
        oa = oracle_quant(a, S.ROWWISE, fmt, S.RNE)
        ob = oracle_quant(b, S.ROWWISE, fmt, S.SR, 3, 3)
        assert oa["texp"] > 0 and ob["texp"] < -20
        c = S.qgemm(upload_oracle_q(oa, fmt), upload_oracle_q(ob, fmt))
        torch.cuda.synchronize()
        check_gemm(c.cpu().numpy().astype(np.float64), oa["xhat"], ob["xhat"], what=f"epilogue fmt={fmt}")


def test_gemm_ldc_and_overwrite():
    fmt = S.NVFP4
    a = synth.gen_matrix((64, 128), seed=3)
    b = synth.gen_matrix((40, 128), seed=4)
    oa, ob = oracle_quant(a, S.ROWWISE, fmt, S.RNE), oracle_quant(b, S.ROWWISE, fmt, S.RNE)
    big = torch.full((64, 64), 7.0, dtype=torch.float32, device="cuda")
    S.qgemm(upload_oracle_q(oa, fmt), upload_oracle_q(ob, fmt), out=big[:, :40])
    torch.cuda.synchronize()
    h = big.cpu().numpy()
    assert np.all(h[:, 40:] == 7.0)                          # untouched beyond N
    check_gemm(h[:, :40].astype(np.float64), oa["xhat"], ob["xhat"], what="ldc")


# Outputs written with ldc > N: the wave sub-tiles inside C take the
# unchecked store (row addresses from ldc), ragged ones the checked store,
# and the columns past N stay untouched. 384 x 320 runs on 64x64 tiles (all
# inside C), 1536 x 2000 on 128x128 tiles (the last tile column is ragged).
@pytest.mark.parametrize("fmt", [S.NVFP4, S.FP8])
@pytest.mark.parametrize("M,N,ldc", [(384, 320, 400), (1536, 2000, 2048)])
def test_gemm_ldc_interior_tiles(fmt, M, N, ldc):
    K = 256
    say(f"gemm ldc interior case fmt={fmt} M={M} N={N} K={K} ldc={ldc}")
    a = synth.gen_matrix((M, K), seed=5)
    b = synth.gen_matrix((N, K), seed=6, std=0.02)
    oa, ob = oracle_quant(a, S.ROWWISE, fmt, S.RNE), oracle_quant(b, S.ROWWISE, fmt, S.SR, 1, 1)
    big = torch.full((M, ldc), 7.0, dtype=torch.float32, device="cuda")
    S.qgemm(upload_oracle_q(oa, fmt), upload_oracle_q(ob, fmt), out=big[:, :N])
    torch.cuda.synchronize()
    h = big.cpu().numpy()
    assert np.all(h[:, N:] == 7.0)
    check_gemm(h[:, :N].astype(np.float64), oa["xhat"], ob["xhat"], what=f"ldc interior fmt={fmt} {M}x{N}")


# Shapes that make the planner pick each kernel and tile: 256x128 for FP8
# and NVFP4, 256x256 for FP8, MX-FP4, BF16 and NVFP4 (K >= 2048 in whole
# pairs of 128-element stages), the register-staged 128x128 kernel for MX-FP4 and BF16, the
# LDS-DMA 128x128 kernel for NVFP4 / FP8 and the 64x64 skinny tiles -- all
# with ragged M and N. Sampled output rows (all columns) against the oracle.
PLAN_CASES = [
    (S.FP8, 4000, 5600, 1024),      # 128x128 (256x128 would leave a last round of 192 tiles)
    (S.NVFP4, 8000, 4000, 512),     # 256x128, 2-stage ring
    (S.NVFP4, 4000, 3900, 8448),    # 256x256, one wave per SIMD (K >= 2048; 66 stages)
    (S.NVFP4, 8000, 4000, 2304),    # the same kernel persistent at K = 2304 (18 stages), 2 tiles per workgroup
    (S.NVFP4, 3800, 17400, 4352),   # the same kernel persistent: 1020 tiles on 256 workgroups (3-4 each),
                                    # ragged edges, loads running on into the next tile between interior
                                    # tiles, 34 stages (the code ring's slots rotate from tile to tile)
    (S.NVFP4, 3800, 17400, 4224),   # 256x128: K >= 2048 in an odd number (33) of stages
    (S.NVFP4, 4000, 5600, 1024),    # 256x128, 2-stage ring
    (S.FP8, 8000, 4000, 512),       # 256x128
    (S.FP8, 1500, 35500, 512),      # 256x256 (834 tiles: 256x128 would leave a last round of 132)
    (S.MXFP4, 8000, 4000, 512),     # 256x256, one wave per SIMD (4 stages: one whole scale group)
    (S.MXFP4, 8000, 4000, 2560),    # 256x256, one wave per SIMD (20 stages: 5 whole scale groups, ring of 3)
    (S.MXFP4, 8000, 4000, 1024),    # persistent, 2 tiles per workgroup: two scale groups, every refill of a
                                    # streaming tile loads the next tile's stages and groups
    (S.MXFP4, 8000, 4000, 1536),    # persistent: three scale groups (the group ring moves on by 3 per tile)
    (S.MXFP4, 8000, 4000, 640),     # 256x256, one wave per SIMD (5 stages: the odd last stage, quad-lane scale loads)
    (S.BF16, 8000, 4000, 256),      # 256x256
    (S.MXFP4, 2000, 1600, 768),     # staged 128x128, 256-element stages
    (S.MXFP4, 2000, 1600, 384),     # staged 128x128, 128-element stages
    (S.BF16, 2000, 1600, 384),      # staged 128x128
    (S.NVFP4, 2000, 1600, 640),     # LDS-DMA 128x128, 2-stage ring (K % 256 != 0)
    (S.NVFP4, 2000, 1600, 768),     # LDS-DMA 128x128, 2-stage ring (K % 256 == 0)
    (S.FP8, 2000, 1600, 640),       # LDS-DMA 128x128, 208 tiles: two-unit stages
    (S.FP8, 3000, 2000, 512),       # LDS-DMA 128x128, 384 tiles: 3-stage ring of single units
    (S.FP8, 4000, 240, 1024),       # 64x64, unsplit, two-unit stages
    (S.NVFP4, 240, 2000, 2048),     # 64x64, K split 4 ways (512 each), two-unit stages
    (S.NVFP4, 240, 2000, 1920),     # 64x64, K split 3 ways (640 each): single-unit stages
]


@pytest.mark.parametrize("fmt,M,N,K", PLAN_CASES)
def test_gemm_each_plan_ragged(fmt, M, N, K):
    say(f"gemm plan case fmt={fmt} M={M} N={N} K={K}")
    a = synth.gen_matrix((M, K), seed=M + K)
    b = synth.gen_matrix((N, K), seed=N + K, std=0.02)
    oa = oracle_quant(a, S.ROWWISE, fmt, S.RNE, 0, 0)
    ob = oracle_quant(b, S.ROWWISE, fmt, S.SR, 1, 1)
    c = S.qgemm(upload_oracle_q(oa, fmt), upload_oracle_q(ob, fmt))
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    edge = [r for r in (0, 255, 256, M - 1) if r < M]     # tile edges that exist at this M
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 96), replace=False), edge]))
    check_gemm(c[rows].cpu().numpy().astype(np.float64), oa["xhat"][rows], ob["xhat"],
               what=f"fmt={fmt} {M}x{N}x{K}")
