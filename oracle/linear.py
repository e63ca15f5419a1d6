"""Quantized linear layer, forward and backward, plus the statistics report.

[SNIP, Fig. 5] and [FP4 All the Way summary, Outline]:
  forward   Y  = Q_rn(X) . Q_rn(W)^T                (K = d_in)
  dgrad     dX = Q_sr(dY) . Q_sr(W^T)^T             (K = d_out)
  wgrad     dW = Q_sr(dY^T) . Q_sr(X^T)^T           (K = T)
Round-to-nearest on the forward operands, stochastic rounding on every
operand of the two backward GEMMs (the "update" pass is read as the weight
gradient GEMM). Both operands of a GEMM use that GEMM's format from the
per-layer plan [SNIP, Abstract]: FP8 or FP4 per layer, BF16 as baseline.

Random-stream tensor ids: 8 * layer_id + role, roles 0..5 =
X fwd, W fwd, dY dgrad, W^T dgrad, dY^T wgrad, X^T wgrad.

Report [FP4 All the Way summary, Outline]: learning with quantized
gradients loses efficiency once the gradient norm drops below about sqrt(3)
times the quantization noise. Reading: noise = ||Q(x) - x|| of the same
tensor, so the flag is sum x^2 < 3 * sum (Q(x)-x)^2.
"""
from __future__ import annotations

import numpy as np

from .quantize import quantize, quantize_colwise, tensor_amax
from .gemm import gemm_q

ROLE_X_FWD, ROLE_W_FWD, ROLE_DY_DGRAD, ROLE_WT_DGRAD, ROLE_DYT_WGRAD, ROLE_XT_WGRAD = range(6)


def tid(layer_id: int, role: int) -> int:
    return 8 * layer_id + role


def linear_fwd(x, w, fmt: int, seed: int = 0, layer_id: int = 0, rows=None, amax_x=None, amax_w=None):
    """x [T, in], w [out, in] (fp32 arrays of bf16 values). rows: optional
    subset of output rows (tokens) to compute; stats always cover the whole
    tensors. amax_x, amax_w: supplied tensor maxima (delayed scaling) or
    None for each tensor's own max."""
    qx = quantize(x, fmt, "rne", seed, tid(layer_id, ROLE_X_FWD), amax=amax_x)
    qw = quantize(w, fmt, "rne", seed, tid(layer_id, ROLE_W_FWD), amax=amax_w)
    y, bound = gemm_q(qx, qw, rows)
    return {"y": y, "bound": bound, "qx": qx, "qw": qw,
            "stats": [qx["stats"], qw["stats"]]}


def linear_bwd(dy, x, w, fmt_dgrad: int, fmt_wgrad: int, seed: int = 0, layer_id: int = 0):
    """dy [T, out], x [T, in], w [out, in]."""
    qdy = quantize(dy, fmt_dgrad, "sr", seed, tid(layer_id, ROLE_DY_DGRAD))
    qwt = quantize_colwise(w, fmt_dgrad, "sr", seed, tid(layer_id, ROLE_WT_DGRAD))
    dx, bdx = gemm_q(qdy, qwt)
    qdyt = quantize_colwise(dy, fmt_wgrad, "sr", seed, tid(layer_id, ROLE_DYT_WGRAD))
    qxt = quantize_colwise(x, fmt_wgrad, "sr", seed, tid(layer_id, ROLE_XT_WGRAD))
    dw, bdw = gemm_q(qdyt, qxt)
    return {"dx": dx, "bound_dx": bdx, "dw": dw, "bound_dw": bdw,
            "q": [qdy, qwt, qdyt, qxt],
            "stats": [qdy["stats"], qwt["stats"], qdyt["stats"], qxt["stats"]]}


def quantize_dual(x, fmt: int, rounding_row: str, rounding_col: str, seed: int, tid_row: int,
                  tid_col: int, amax=None):
    """Both layouts of one tensor [SNIP, Fig. 5: X, W and dY each feed two
    GEMMs, along different dimensions]: by definition the row-wise and the
    column-wise quantization of x, each with its own rounding and stream."""
    return (quantize(x, fmt, rounding_row, seed, tid_row, amax=amax),
            quantize_colwise(x, fmt, rounding_col, seed, tid_col, amax=amax))


def linear_fwd_save(x, w, fmt: int, seed: int = 0, layer_id: int = 0, amax_x=None, amax_w=None):
    """Forward plus the backward operands built from x and w, in the
    layer's one format: what linear_fwd computes, and the column-wise SR
    operands W^T (dgrad B) and X^T (wgrad B) that linear_bwd builds. With
    supplied maxima both layouts of a tensor use the same one."""
    f = linear_fwd(x, w, fmt, seed, layer_id, amax_x=amax_x, amax_w=amax_w)
    qwt = quantize_colwise(w, fmt, "sr", seed, tid(layer_id, ROLE_WT_DGRAD), amax=amax_w)
    qxt = quantize_colwise(x, fmt, "sr", seed, tid(layer_id, ROLE_XT_WGRAD), amax=amax_x)
    f.update(qwt=qwt, qxt=qxt, stats=[f["qx"]["stats"], f["qw"]["stats"], qwt["stats"], qxt["stats"]])
    return f


def linear_bwd_saved(dy, qwt: dict, qxt: dict, fmt: int, seed: int = 0, layer_id: int = 0, amax_dy=None):
    """Backward from saved W^T and X^T operands: dY quantized both ways
    (with the supplied max amax_dy, or its own)."""
    qdy = quantize(dy, fmt, "sr", seed, tid(layer_id, ROLE_DY_DGRAD), amax=amax_dy)
    qdyt = quantize_colwise(dy, fmt, "sr", seed, tid(layer_id, ROLE_DYT_WGRAD), amax=amax_dy)
    dx, bdx = gemm_q(qdy, qwt)
    dw, bdw = gemm_q(qdyt, qxt)
    return {"dx": dx, "bound_dx": bdx, "dw": dw, "bound_dw": bdw, "q": [qdy, qdyt],
            "stats": [qdy["stats"], qdyt["stats"]]}


def report(stats: dict) -> dict:
    """Derived per-tensor report from one statistics record."""
    e2, x2 = stats["sum_err2"], stats["sum_x2"]
    rel = e2 / x2 if x2 > 0 else (0.0 if e2 == 0 else np.inf)
    ratio = np.sqrt(x2) / np.sqrt(e2) if e2 > 0 else np.inf
    return {"rel_mse": rel, "norm_ratio": ratio,
            "below_sqrt3": bool(x2 < 3.0 * e2), "amax": stats["amax"],
            "n_nonfinite": stats["n_nonfinite"]}


def fp4_flop_share(layers, plan, tokens: int) -> float:
    """Share of the GEMM FLOPs of a block that run in an FP4 format."""
    tot = fp4 = 0
    for layer, fmt in zip(layers, plan):
        f = 3 * 2 * tokens * layer.d_in * layer.d_out
        tot += f
        if fmt in (2, 3):
            fp4 += f
    return fp4 / tot
