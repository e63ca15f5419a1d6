"""snip_qgemm_qout: a GEMM whose launch also quantizes its fp32 output
row-wise (NVFP4 or FP8, nearest or stochastic, tensor scale from a supplied
max) ["SNIP", Fig. 5: a layer's output is the next layer's quantized
operand].

Bit-exact parity needs the oracle and the GPU to quantize the same fp32
values, and a GEMM's fp32 output depends on its summation order. The
operands here are therefore built so that every product and partial sum is
exactly representable: E2M1-grid values with a +-6 in every 16-block (so
every NVFP4 block scale is the same power of two and the quantized operand
equals its input), or small integers for FP8. Then C is the same exact
fp32 number in any order: the oracle's fp64 product equals the GPU's C
bit for bit (checked), and the oracle quantizes its own C. Codes, scales
and the tensor exponent are compared bit-exactly, statistics within 1e-5.
The shapes select every GEMM kernel the entry point runs (256x256, 256x128,
128x128 and 64x64 tiles, and split-K, where the reduction kernel
quantizes). Realistic (Gaussian) operands check C against the 1e-5 bound.
"""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from oracle import quantize as OQ
from parity import RND, check_gemm, compare_codes, compare_stats, gpu_codes, oracle_chunked, say

pytestmark = pytest.mark.gpu

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def exact_operand(rows, k, fmt, seed):
    """bf16 operand whose quantization in `fmt` is exact and whose products
    sum exactly: NVFP4: E2M1-grid values, each 16-block holding a +-6 (one
    block scale for the whole tensor); FP8: integers in [-8, 8] with an 8."""
    rng = np.random.default_rng(seed)
    if fmt == S.NVFP4:
        v = E2M1_GRID[rng.integers(0, 8, size=(rows, k))] * rng.choice([-1.0, 1.0], size=(rows, k))
        pos = rng.integers(0, 16, size=(rows, k // 16))
        v.reshape(rows, k // 16, 16)[np.arange(rows)[:, None], np.arange(k // 16)[None, :], pos] = 6.0
    else:
        v = rng.integers(-8, 9, size=(rows, k)).astype(np.float32)
        v[:, 0] = 8.0
    return synth.to_bf16(v.astype(np.float32))


# (operand format, M, N, K, output format, rounding, amax factor): the shapes
# select 256x128 (NVFP4, FP8), 256x256 (FP8, and NVFP4 for K >= 2048 in
# pairs of 128-element stages),
# 128x128, 64x64 unsplit and split-K plans, ragged in M.
CASES = [
    (S.NVFP4, 4000, 4096, 256, S.NVFP4, S.RNE, 1.0),      # 256x128
    (S.NVFP4, 4000, 3904, 8448, S.NVFP4, S.SR, 1.0),      # 256x256, one wave per SIMD (66 stages)
    (S.NVFP4, 4000, 3904, 2304, S.FP8, S.RNE, 1.0),       # the same at K = 2304 (18 stages)
    (S.NVFP4, 2000, 1600, 256, S.FP8, S.SR, 1.0),         # 128x128
    (S.NVFP4, 1000, 1200, 512, S.NVFP4, S.SR, 0.5),       # 64x64 unsplit; stale max below: saturation
    (S.NVFP4, 240, 2000, 2048, S.NVFP4, S.RNE, 4.0),      # 64x64, K split 4 ways: quantized in the reduction
    (S.NVFP4, 240, 2000, 2048, S.FP8, S.SR, 1.0),         # split-K, FP8 output, stochastic
    (S.FP8, 4096, 4096, 256, S.FP8, S.RNE, 1.0),          # 256x128
    (S.FP8, 1500, 35520, 256, S.NVFP4, S.SR, 1.0),        # 256x256
    (S.FP8, 2000, 1600, 640, S.NVFP4, S.RNE, 2.0),        # 128x128, two-unit stages
    (S.FP8, 3000, 2000, 512, S.FP8, S.SR, 1.0),           # 128x128, three-stage ring
    (S.FP8, 4000, 240, 1024, S.NVFP4, S.RNE, 1.0),        # 64x64 unsplit
    (S.FP8, 256, 2048, 4096, S.NVFP4, S.SR, 1.0),         # 64x64 split-K
]


@pytest.mark.parametrize("fmt,M,N,K,ofmt,rnd,afac", CASES)
def test_qgemm_qout_bit_exact(fmt, M, N, K, ofmt, rnd, afac):
    seed, tid = 7, 8 * 3 + 2
    say(f"qgemm_qout case fmt={fmt} M={M} N={N} K={K} out={ofmt} rounding={rnd} amax x{afac}")
    a = exact_operand(M, K, fmt, 11 + M)
    b = exact_operand(N, K, fmt, 13 + N)
    qa, _ = S.quantize(a.cuda(), S.ROWWISE, fmt, S.RNE, with_stats=False)
    qb, _ = S.quantize(b.cuda(), S.ROWWISE, fmt, S.RNE, with_stats=False)
    oa = OQ.quantize(synth.bf16_to_f32(a), fmt, "rne")
    ob = OQ.quantize(synth.bf16_to_f32(b), fmt, "rne")
    assert np.array_equal(oa["xhat"], synth.bf16_to_f32(a)) and np.array_equal(ob["xhat"], synth.bf16_to_f32(b))
    c_ref = oa["xhat"] @ ob["xhat"].T                                # exact: integers / quarters
    c32 = c_ref.astype(np.float32)
    assert np.array_equal(c32.astype(np.float64), c_ref)
    amax = np.float32(OQ.tensor_amax(c32) * afac)
    c, q, st = S.qgemm_qout(qa, qb, ofmt, torch.tensor([amax], device="cuda"), rnd, seed, tid)
    torch.cuda.synchronize()
    cg = c.cpu().numpy()
    mism = np.argwhere(cg != c32)
    assert mism.size == 0, f"C differs from the exact product at {mism[:4].tolist()}"
    o = oracle_chunked(c32, ofmt, S.ROWWISE, rnd, seed, tid, amax=amax, keep=True)
    compare_codes(gpu_codes(q), o, ofmt, what=f"qout fmt={fmt} {M}x{N}x{K} -> {ofmt}")
    compare_stats(S.decode_stats(st)[0], o["stats"], what="qout stats")


def test_qgemm_qout_ldc_and_realistic_operands():
    """Gaussian NVFP4 operands (the TinyLlama Q projection, 4096x2048x2048)
    written into a wider C (ldc > N): C within 1e-5 sum|a||b| of the oracle
    on sampled rows, columns past N untouched, and the quantized output's
    tensor exponent that of the supplied max."""
    M, N, K, ldc = 4096, 2048, 2048, 2048 + 64
    say(f"qgemm_qout realistic case {M}x{N}x{K} ldc={ldc}")
    a = synth.gen_matrix((M, K), seed=31)
    b = synth.gen_matrix((N, K), seed=32, std=0.02)
    qa, _ = S.quantize(a.cuda(), S.ROWWISE, S.NVFP4, S.RNE, with_stats=False)
    qb, _ = S.quantize(b.cuda(), S.ROWWISE, S.NVFP4, S.RNE, with_stats=False)
    big = torch.full((M, ldc), 5.0, dtype=torch.float32, device="cuda")
    amax = np.float32(3.0)
    c, q, st = S.qgemm_qout(qa, qb, S.NVFP4, torch.tensor([amax], device="cuda"), S.RNE, 0, 1, c=big[:, :N])
    c_plain = S.qgemm(qa, qb)
    torch.cuda.synchronize()
    h = big.cpu().numpy()
    assert np.all(h[:, N:] == 5.0)
    assert torch.equal(big[:, :N], c_plain), "C differs from snip_qgemm's"
    oa = OQ.quantize(synth.bf16_to_f32(a), S.NVFP4, "rne")
    ob = OQ.quantize(synth.bf16_to_f32(b), S.NVFP4, "rne")
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(M, 64, replace=False), [0, 255, 256, M - 1]]))
    check_gemm(h[rows, :N].astype(np.float64), oa["xhat"][rows], ob["xhat"], what="qout realistic C")
    assert int(q.texp.item()) == OQ.pow2_tensor_exp(amax, OQ.NVFP4_RANGE)
    g = S.decode_stats(st)[0]
    assert g["amax"] == float(np.max(np.abs(c_plain.cpu().numpy())))
