"""Pins for the oracle's GEMM and linear composition.

  * fp64 GEMM of dequantized operands against exact rational dot products
    (fractions.Fraction) on tiny tensors;
  * a representable operand pair gives a quantized GEMM equal to the plain
    fp64 product of the inputs;
  * linearity in each operand for values that stay representable;
  * linear forward/backward composition: each output is the reference GEMM
    of the operands quantized with the right rounding and tensor id; the
    backward GEMMs approach the exact gradients as the formats get finer.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm as G
from oracle import linear as L
from oracle import quantize as Q
from oracle import formats as F


def test_gemm_matches_exact_rationals():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    w = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    qa = Q.quantize(x, Q.NVFP4, "rne")
    qb = Q.quantize(w, Q.NVFP4, "sr", seed=1, tensor_id=1)
    c, bound = G.gemm_q(qa, qb)
    A, B = qa["xhat"], qb["xhat"]
    for i in range(16):
        for j in range(8):
            exact = sum(Fraction(float(A[i, k])) * Fraction(float(B[j, k])) for k in range(128))
            babs = sum(abs(Fraction(float(A[i, k])) * Fraction(float(B[j, k]))) for k in range(128))
            assert abs(Fraction(float(c[i, j])) - exact) <= Fraction(1, 10 ** 12) * babs
            assert float(babs) == pytest.approx(bound[i, j], rel=1e-14)


def test_representable_gemm_equals_plain_product():
    rng = np.random.default_rng(1)
    codes_a = rng.integers(0, 16, (32, 64)).astype(np.uint8)
    codes_b = rng.integers(0, 16, (16, 64)).astype(np.uint8)
    codes_a[:, 0::16] = 7                 # a +-6 in every 16-block: exact block scales
    codes_b[:, 0::16] = 15
    a = (F.e2m1_decode(codes_a) * 0.5).astype(np.float32)
    b = (F.e2m1_decode(codes_b) * 4.0).astype(np.float32)
    for fmt in (Q.MXFP4, Q.NVFP4):
        qa = Q.quantize(a, fmt, "rne")
        qb = Q.quantize(b, fmt, "sr", seed=2)
        c, _ = G.gemm_q(qa, qb)
        assert np.array_equal(c, a.astype(np.float64) @ b.astype(np.float64).T)


def test_gemm_linearity():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((8, 32))
    b1 = rng.standard_normal((4, 32))
    b2 = rng.standard_normal((4, 32))
    c1, _ = G.gemm_ref(a, b1)
    c2, _ = G.gemm_ref(a, b2)
    c12, _ = G.gemm_ref(a, b1 + b2)
    assert np.allclose(c12, c1 + c2, rtol=1e-12, atol=1e-12)
    ca, _ = G.gemm_ref(2 * a, b1)
    assert np.array_equal(ca, 2 * c1)


def test_check_bound():
    c_ref = np.array([[1.0, -2.0]])
    bound = np.array([[10.0, 10.0]])
    ok, worst = G.check(c_ref + 9e-5, c_ref, bound)
    assert ok and worst == pytest.approx(9e-6)
    ok, _ = G.check(c_ref + 2e-4, c_ref, bound)
    assert not ok


def test_linear_composition_and_tensor_ids():
    rng = np.random.default_rng(3)
    T, din, dout = 32, 64, 48
    x = rng.standard_normal((T, din)).astype(np.float32)
    w = (rng.standard_normal((dout, din)) * 0.02).astype(np.float32)
    dy = (rng.standard_normal((T, dout)) * 1e-3).astype(np.float32)
    fwd = L.linear_fwd(x, w, Q.NVFP4, seed=4, layer_id=3)
    qx = Q.quantize(x, Q.NVFP4, "rne", 4, 24)
    qw = Q.quantize(w, Q.NVFP4, "rne", 4, 25)
    assert np.array_equal(fwd["y"], qx["xhat"] @ qw["xhat"].T)
    bwd = L.linear_bwd(dy, x, w, Q.FP8, Q.NVFP4, seed=4, layer_id=3)
    qdy = Q.quantize(dy, Q.FP8, "sr", 4, 26)
    qwt = Q.quantize(np.ascontiguousarray(w.T), Q.FP8, "sr", 4, 27)
    assert np.array_equal(bwd["dx"], qdy["xhat"] @ qwt["xhat"].T)
    qdyt = Q.quantize(np.ascontiguousarray(dy.T), Q.NVFP4, "sr", 4, 28)
    qxt = Q.quantize(np.ascontiguousarray(x.T), Q.NVFP4, "sr", 4, 29)
    assert np.array_equal(bwd["dw"], qdyt["xhat"] @ qxt["xhat"].T)


def test_backward_approaches_exact_gradients():
    rng = np.random.default_rng(5)
    T, din, dout = 64, 64, 32
    x = rng.standard_normal((T, din)).astype(np.float32)
    w = (rng.standard_normal((dout, din)) * 0.02).astype(np.float32)
    dy = (rng.standard_normal((T, dout)) * 1e-3).astype(np.float32)
    dx_true = dy.astype(np.float64) @ w.astype(np.float64)
    dw_true = dy.astype(np.float64).T @ x.astype(np.float64)
    errs = []
    for fmt in (Q.NVFP4, Q.FP8, Q.BF16):
        b = L.linear_bwd(dy, x, w, fmt, fmt, seed=0, layer_id=0)
        errs.append((np.linalg.norm(b["dx"] - dx_true) / np.linalg.norm(dx_true),
                     np.linalg.norm(b["dw"] - dw_true) / np.linalg.norm(dw_true)))
    assert errs[2] == (0.0, 0.0)
    assert errs[1][0] < errs[0][0] and errs[1][1] < errs[0][1]
    assert errs[0][0] < 0.3 and errs[0][1] < 0.3


def test_report_sqrt3_flag():
    rep = L.report({"sum_err2": 1.0, "sum_x2": 2.9, "amax": 1.0, "n_nonfinite": 0})
    assert rep["below_sqrt3"] and rep["norm_ratio"] == pytest.approx(np.sqrt(2.9))
    rep = L.report({"sum_err2": 1.0, "sum_x2": 3.1, "amax": 1.0, "n_nonfinite": 0})
    assert not rep["below_sqrt3"]


def test_fp4_flop_share_plans():
    import synth
    wl = synth.WORKLOADS["llama7b"]
    share = L.fp4_flop_share(wl.layers, wl.plan, wl.tokens)
    assert share == pytest.approx(0.8342, abs=1e-4)
    wl = synth.WORKLOADS["llama70b"]
    assert L.fp4_flop_share(wl.layers, wl.plan, wl.tokens) == 1.0
