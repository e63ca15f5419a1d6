"""Reference GEMM on dequantized operands, and the parity bound.

[SNIP, Fig. 5]: each linear layer runs its forward and backward GEMMs on the
quantized operands. Every GEMM here has the form C[M, N] = A[M, K] . B[N, K]^T
with both operands laid out along K. The reference dequantizes both operands
exactly into fp64 and multiplies them in fp64; the bound for an output
element is sum_k |A[m,k]| |B[n,k]|, and a device result passes when
|C_dev - C_ref| <= 1e-5 * bound elementwise.
"""
from __future__ import annotations

import numpy as np


def gemm_ref(a_hat: np.ndarray, b_hat: np.ndarray):
    """C = A . B^T and the elementwise bound sum |A||B|, both fp64."""
    a = np.asarray(a_hat, dtype=np.float64)
    b = np.asarray(b_hat, dtype=np.float64)
    if a.shape[1] != b.shape[1]:
        raise ValueError("K mismatch")
    c = a @ b.T
    bound = np.abs(a) @ np.abs(b).T
    return c, bound


def gemm_q(qa: dict, qb: dict, rows=None):
    """Reference product of two quantized operands (oracle.quantize output).
    rows: optional subset of A rows to compute."""
    a = qa["xhat"] if rows is None else qa["xhat"][rows]
    return gemm_ref(a, qb["xhat"])


def check(c_dev: np.ndarray, c_ref: np.ndarray, bound: np.ndarray, tol: float = 1e-5):
    """Returns (ok, worst ratio |diff| / bound)."""
    diff = np.abs(np.asarray(c_dev, dtype=np.float64) - c_ref)
    lim = tol * bound
    ok = bool(np.all(diff <= lim))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, diff / bound, np.where(diff > 0, np.inf, 0.0))
    return ok, float(np.max(ratio)) if ratio.size else 0.0


def flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k
