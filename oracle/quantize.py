"""Quantizers: NVFP4 (16 x E2M1 + E4M3 block scale), FP8-E4M3 per tensor,
MX-style FP4 (32 x E2M1 + E8M0 block scale), with round-to-nearest-even or
stochastic rounding, plus the per-tensor statistics.

[FP4 All the Way summary, Outline]: blocks of 16 E2M1 values share an E4M3
scale; forward operands use round-to-nearest, back-propagation and update
operands use stochastic rounding. [SNIP, Abstract]: statistics of
activations and gradients are collected to judge the precision loss; each
pass here records sum (Q(x)-x)^2, sum x^2 and max|x|.

Readings (the pages do not fix these):
  * Blocks run along the reduction dimension K of the GEMM that consumes the
    operand, so every block scale factors out of the dot product. Row-wise
    quantization of [R, C] blocks along C; column-wise quantization is the
    row-wise quantization of the transpose.
  * NVFP4 carries a power-of-two tensor scale S = 2^eS above the E4M3 block
    scales: the smallest power of two with max|x| / S <= 6 * 448, so that no
    block scale saturates and small-magnitude tensors (gradients ~1e-3,
    weights ~0.02) keep their E4M3 block scales in the normal range.
  * Block scale: s_b = E4M3_RNE(fp32(a_b / 6)) with a_b = max|x / S| over the
    block, computed in the scaled domain x' = ldexp(x, -eS).
  * Element: r = fp32(x' * fp32(1 / s_b)) (one reciprocal per block, one
    multiply per element), then E2M1 rounding of r. A block whose scale code
    is 0 gets magnitude-0 codes that keep the sign bit of x.
  * FP8: per-tensor power-of-two scale, smallest with max|x| / S <= 448;
    r = ldexp(x, -eS), then E4M3 rounding with saturation at 448.
  * MX: per-32 E8M0 scale X_b = floor(log2 a_b) - 2 (OCP rule, E2M1 largest
    exponent 2), clamped to [-127, 127], X_b = -127 for a zero block;
    r = ldexp(x, -X_b); values in (6, 8) saturate to 6.
  * FP4 design-space variants [FP4 All the Way summary, Outline: block size,
    scaling format and rounding were explored]: E2M1 codes with a block of
    16 or 32 and an E4M3, E8M0 or BF16 block scale. E4M3 scales follow the
    NVFP4 rules with any block (tensor scale, s = E4M3_RNE(a_b / 6)); E8M0
    scales follow the MX rule with any block; a BF16 scale is
    s = bf16_RNE(fp32(a_b / 6)) of the raw block max (bf16 has the range, so
    no tensor scale), then r = fp32(x * fp32(1 / s)). NVFP4 is the (16,
    E4M3) variant and MX-FP4 the (32, E8M0) one.
  * The max|x| statistic is that of the tensor quantized, also when the
    tensor scale comes from a supplied max (delayed scaling: the supplied
    max is an earlier step's statistic, so each step must report its own).
    For a caller quantizing a subset of a larger tensor's rows it is the
    subset's max, like the sums.
  * Non-finite inputs lie outside the contract: they are counted, the tensor
    max ignores them, the statistics sum only finite elements, and the codes
    of a block holding one are unspecified (reported in `bad_blocks`).
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .philox import r16 as philox_r16

BF16, FP8, NVFP4, MXFP4 = 0, 1, 2, 3
# design-space variants of FP4 (quantizer only): E2M1 with (block, scale)
FP4_E4M3_B32, FP4_E8M0_B16, FP4_BF16_B16, FP4_BF16_B32 = 4, 5, 6, 7
FP4_VARIANT = {NVFP4: (16, "e4m3"), MXFP4: (32, "e8m0"), FP4_E4M3_B32: (32, "e4m3"),
               FP4_E8M0_B16: (16, "e8m0"), FP4_BF16_B16: (16, "bf16"), FP4_BF16_B32: (32, "bf16")}
BLOCK = {FP8: 1, BF16: 1, **{f: v[0] for f, v in FP4_VARIANT.items()}}
NVFP4_RANGE = 6.0 * 448.0   # largest E2M1 magnitude x largest E4M3 scale
FP8_RANGE = 448.0


def tensor_amax(x: np.ndarray) -> np.float32:
    """max |x| over the finite elements (0 if there are none)."""
    x = np.asarray(x, dtype=np.float32)
    fin = np.isfinite(x)
    if not fin.any():
        return np.float32(0.0)
    return np.float32(np.max(np.abs(np.where(fin, x, 0.0))))


def pow2_tensor_exp(amax: float, limit: float) -> int:
    """Smallest integer e with amax * 2^-e <= limit (0 when amax == 0)."""
    a = float(amax)
    if a == 0.0:
        return 0
    e = int(np.frexp(a)[1]) - int(np.frexp(limit)[1]) - 2   # a safe under-estimate
    while np.ldexp(a, -e) > limit:
        e += 1
    while np.ldexp(a, -(e - 1)) <= limit:
        e -= 1
    return e


def _draws(rounding: str, seed: int, tensor_id: int, row_ids: np.ndarray, K: int):
    if rounding == "rne":
        return None
    idx = row_ids.astype(np.uint64)[:, None] * np.uint64(K) + np.arange(K, dtype=np.uint64)[None, :]
    return philox_r16(seed, tensor_id, idx)


def _stats(x: np.ndarray, xhat: np.ndarray, amax: float) -> dict:
    x64 = x.astype(np.float64)
    fin = np.isfinite(x64)
    xf = np.where(fin, x64, 0.0)
    err = np.where(fin, xhat - xf, 0.0)
    return {
        "sum_err2": float(np.sum(err * err)),
        "sum_x2": float(np.sum(xf * xf)),
        "amax": float(amax),
        "n_nonfinite": int(np.count_nonzero(~fin)),
    }


def quantize(x: np.ndarray, fmt: int, rounding: str = "rne", seed: int = 0,
             tensor_id: int = 0, amax=None, row_ids=None) -> dict:
    """Row-wise quantization of x [R, K] (fp32 array holding bf16 values).

    rounding: "rne" or "sr". amax: tensor max to use instead of max|x| (lets
    a caller quantize a subset of rows of a larger tensor). row_ids: global
    output-row indices of the given rows, for the random-stream element index.
    Returns codes (one per element), packed bytes, scales, tensor exponent,
    the fp64 dequantized tensor and the statistics.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    R, K = x.shape
    blk = BLOCK[fmt]
    if K % blk:
        raise ValueError(f"K={K} not a multiple of the block {blk}")
    if row_ids is None:
        row_ids = np.arange(R)
    row_ids = np.asarray(row_ids)
    A = tensor_amax(x) if amax is None else np.float32(amax)
    fin = np.isfinite(x)
    xc = np.where(fin, x, np.float32(0.0)).astype(np.float32)
    draws = _draws(rounding, seed, tensor_id, row_ids, K)
    out = {"format": fmt, "rows": R, "k": K, "amax": float(A)}

    if fmt == BF16:
        out.update(codes=None, packed=None, scales=None, texp=0,
                   xhat=x.astype(np.float64))
        out["stats"] = _stats(x, out["xhat"], tensor_amax(x))
        out["bad_blocks"] = ~fin
        return out

    if fmt == FP8:
        eS = pow2_tensor_exp(A, FP8_RANGE)
        r = np.ldexp(xc, -eS).astype(np.float32)
        codes = F.e4m3_encode(r, rounding, draws)
        xhat = np.ldexp(F.e4m3_decode(codes), eS)
        out.update(codes=codes, packed=codes, scales=None, texp=eS, xhat=xhat)
        out["stats"] = _stats(x, xhat, tensor_amax(x))
        out["bad_blocks"] = ~fin
        return out

    nb = K // blk
    sign = np.signbit(xc)
    kind = FP4_VARIANT[fmt][1] if fmt in FP4_VARIANT else None
    if kind == "e4m3":
        eS = pow2_tensor_exp(A, NVFP4_RANGE)
        xs = np.ldexp(xc, -eS).astype(np.float32)                     # x'
        a_b = np.max(np.abs(xs.reshape(R, nb, blk)), axis=2)           # fp32
        t_b = (a_b / np.float32(6.0)).astype(np.float32)               # fp32 divide
        s_code = F.e4m3_encode(t_b, "rne")
        s_hat = F.e4m3_decode(s_code)                                  # exact
        live = s_hat > 0
        s32 = np.where(live, s_hat, 1.0).astype(np.float32)
        inv = (np.float32(1.0) / s32).astype(np.float32)               # fp32 reciprocal
        r = (xs.reshape(R, nb, blk) * inv[:, :, None]).astype(np.float32)
        scale_val = s_hat                                              # per block
        texp = eS
    elif kind == "e8m0":
        a_b = np.max(np.abs(xc.reshape(R, nb, blk)), axis=2).astype(np.float64)
        fl = np.frexp(np.where(a_b > 0, a_b, 1.0))[1] - 1              # floor(log2 a_b)
        X = np.where(a_b > 0, fl - 2, -127)
        X = np.clip(X, -127, 127).astype(np.int64)
        s_code = (X + 127).astype(np.uint8)
        live = a_b > 0
        r = np.ldexp(xc.reshape(R, nb, blk), -X[:, :, None]).astype(np.float32)
        scale_val = np.ldexp(1.0, X)
        texp = 0
    elif kind == "bf16":
        a_b = np.max(np.abs(xc.reshape(R, nb, blk)), axis=2)              # fp32
        t_b = (a_b / np.float32(6.0)).astype(np.float32)                  # fp32 divide
        s_code = F.bf16_scale_encode(t_b)
        s_hat = F.bf16_decode(s_code)                                     # exact
        live = s_hat > 0
        s32 = np.where(live, s_hat, 1.0).astype(np.float32)
        inv = (np.float32(1.0) / s32).astype(np.float32)                  # fp32 reciprocal
        r = (xc.reshape(R, nb, blk) * inv[:, :, None]).astype(np.float32)
        scale_val = s_hat
        texp = 0
    else:
        raise ValueError(f"unknown format {fmt}")

    r = np.where(live[:, :, None], r, np.float32(0.0)).reshape(R, K)
    codes = F.e2m1_encode(r, rounding, draws)
    # dead blocks: magnitude 0 with the sign bit of x
    dead = np.repeat(~live, blk, axis=1)
    codes = np.where(dead, (sign.astype(np.uint8) << 3), codes).astype(np.uint8)
    q = F.e2m1_decode(codes)
    xhat = np.ldexp(q * np.repeat(scale_val, blk, axis=1), texp)
    bad = np.repeat(~fin.reshape(R, nb, blk).all(axis=2), blk, axis=1)
    scales = s_code.astype(np.uint16 if kind == "bf16" else np.uint8)
    out.update(codes=codes, packed=F.pack_nibbles(codes), scales=scales,
               texp=texp, xhat=xhat, bad_blocks=bad)
    out["stats"] = _stats(x, xhat, tensor_amax(x))
    return out


def quantize_colwise(x: np.ndarray, fmt: int, rounding: str = "rne", seed: int = 0,
                     tensor_id: int = 0, amax=None, col_ids=None) -> dict:
    """Column-wise quantization of x [R, C]: blocks run along R and the output
    is laid out [C, R] (row-wise quantization of the transpose)."""
    x = np.asarray(x, dtype=np.float32)
    A = tensor_amax(x) if amax is None else amax
    xt = np.ascontiguousarray(x.T) if col_ids is None else np.ascontiguousarray(x[:, col_ids].T)
    return quantize(xt, fmt, rounding, seed, tensor_id, amax=A, row_ids=col_ids)


def dequantize(q: dict) -> np.ndarray:
    return q["xhat"]
