"""Helpers shared by the GPU parity tests: run a step on the HIP path through
the C ABI, run the same step in the oracle, compare.

Bars: codes, scales, tensor exponents and stochastic-rounding decisions are
compared bit-exactly; GEMM outputs within 1e-5 * sum_k |a_k||b_k| per element;
statistics within 1e-5 of the matching sum (sum x^2 for sum x^2, sum err^2 for
sum err^2), max|x| and the non-finite count exactly.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import synth
from oracle import gemm as OG
from oracle import quantize as OQ

import sub_byte_mixed_amd as S

TOL = 1e-5
RND = {S.RNE: "rne", S.SR: "sr"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f32(x_bf16: torch.Tensor) -> np.ndarray:
    return synth.bf16_to_f32(x_bf16.cpu())


def oracle_quant(x_bf16, layout, fmt, rounding, seed=0, tid=0, amax=None, rows=None):
    x = f32(x_bf16)
    if layout == S.ROWWISE:
        if rows is None:
            return OQ.quantize(x, fmt, RND[rounding], seed, tid, amax=amax)
        A = OQ.tensor_amax(x) if amax is None else amax
        return OQ.quantize(x[rows], fmt, RND[rounding], seed, tid, amax=A, row_ids=rows)
    return OQ.quantize_colwise(x, fmt, RND[rounding], seed, tid, amax=amax, col_ids=rows)


def gpu_codes(q: S.QuantizedTensor) -> dict:
    R, K = q.rows, q.k
    out = {"texp": int(q.texp.cpu().item())}
    c = q.codes.cpu().numpy()
    if q.format in S.FP4_LAYOUT:
        out["packed"] = c.reshape(R, K // 2)
        blk, kind = S.FP4_LAYOUT[q.format]
        sc = q.scales.cpu().numpy()
        out["scales"] = (sc.view(np.uint16) if kind == "bf16" else sc).reshape(R, K // blk)
    elif q.format == S.FP8:
        out["codes"] = c.reshape(R, K)
    else:
        out["codes"] = c.view(np.uint16).reshape(R, K)
    return out


def compare_codes(g: dict, o: dict, fmt: int, rows=None, what=""):
    """Bit-exact comparison of one quantized operand (optionally only the
    given output rows of the GPU result). Blocks holding non-finite inputs
    are excluded (their codes are unspecified)."""
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    if fmt in (S.NVFP4, S.FP8, S.FP4_E4M3_B32):
        assert g["texp"] == o["texp"], f"{what}: tensor exponent {g['texp']} != {o['texp']}"
    bad = o.get("bad_blocks")
    if fmt in S.FP4_LAYOUT:
        gp = sel(g["packed"])
        op = o["packed"]
        if bad is not None and bad.any():
            keep = ~bad.reshape(bad.shape[0], -1, 2).any(axis=2)
            gp, op = gp[keep], op[keep]
        mism = np.argwhere(gp != op)
        assert mism.size == 0, f"{what}: {len(mism)} code bytes differ, first at {mism[:4].tolist()}"
        blk = S.FP4_LAYOUT[fmt][0]
        gs, os_ = sel(g["scales"]), o["scales"]
        if bad is not None and bad.any():
            keepb = ~bad[:, ::blk]
            gs, os_ = gs[keepb], os_[keepb]
        assert np.array_equal(gs, os_), f"{what}: scales differ"
    elif fmt == S.FP8:
        gc, oc = sel(g["codes"]), o["codes"]
        if bad is not None and bad.any():
            gc, oc = gc[~bad], oc[~bad]
        mism = np.argwhere(gc != oc)
        assert mism.size == 0, f"{what}: {len(mism)} fp8 codes differ, first at {mism[:4].tolist()}"


def compare_stats(gs: dict, os_: dict, what="", check_err=True):
    assert gs["n_nonfinite"] == os_["n_nonfinite"], f"{what}: non-finite {gs['n_nonfinite']} != {os_['n_nonfinite']}"
    assert gs["amax"] == np.float32(os_["amax"]), f"{what}: amax {gs['amax']} != {os_['amax']}"
    assert abs(gs["sum_x2"] - os_["sum_x2"]) <= TOL * os_["sum_x2"] + 1e-300, \
        f"{what}: sum_x2 {gs['sum_x2']} vs {os_['sum_x2']}"
    if check_err:
        assert abs(gs["sum_err2"] - os_["sum_err2"]) <= TOL * os_["sum_err2"] + 1e-300, \
            f"{what}: sum_err2 {gs['sum_err2']} vs {os_['sum_err2']}"


def upload_oracle_q(o: dict, fmt: int, device="cuda") -> S.QuantizedTensor:
    """Oracle-quantized operand -> device buffers in the ABI layout."""
    R, K = o["rows"], o["k"]
    if fmt in (S.NVFP4, S.MXFP4):
        codes = torch.from_numpy(np.ascontiguousarray(o["packed"]).reshape(-1)).to(device)
        scales = torch.from_numpy(np.ascontiguousarray(o["scales"]).reshape(-1)).to(device)
    elif fmt == S.FP8:
        codes = torch.from_numpy(np.ascontiguousarray(o["codes"]).reshape(-1)).to(device)
        scales = None
    else:
        bits = np.ascontiguousarray(o["xhat"].astype(np.float32)).view(np.uint32) >> 16
        codes = torch.from_numpy(bits.astype(np.uint16).view(np.uint8).reshape(-1)).to(device)
        scales = None
    texp = torch.tensor([o.get("texp", 0)], dtype=torch.int32, device=device)
    return S.QuantizedTensor(fmt, R, K, device, codes=codes, scales=scales, texp=texp)


def check_gemm(c_gpu: np.ndarray, a_hat: np.ndarray, b_hat: np.ndarray, what=""):
    c_ref, bound = OG.gemm_ref(a_hat, b_hat)
    ok, worst = OG.check(c_gpu, c_ref, bound, TOL)
    if not ok:
        diff = np.abs(c_gpu - c_ref)
        i = np.unravel_index(np.argmax(diff - TOL * bound), diff.shape)
        raise AssertionError(f"{what}: GEMM outside 1e-5*sum|a||b| (worst ratio {worst:.3e}) at {i}: "
                             f"gpu {c_gpu[i]} ref {c_ref[i]} bound {bound[i]}")
    return worst


# ---------------------------------------------------------------- full-tensor oracle, in chunks
# The oracle's quantizers are numpy element-wise code: a large tensor is
# quantized in chunks of output rows (each with the whole tensor's max and
# its global row indices, so every code, scale and random draw is the one
# the whole-tensor call gives), on a pool of threads (numpy releases the
# interpreter lock inside its array loops). The chunks' statistics are summed
# in fp64; their codes and dequantized values are concatenated when asked for.
_POOL = None


def oracle_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=oracle_threads())
    return _POOL


def oracle_chunked(t32: np.ndarray, fmt: int, layout: int, rounding: int, seed: int, tid: int,
                   amax=None, keep: bool = False, chunk_elems: int = 1 << 21) -> dict:
    """Oracle quantization of the whole tensor t32 [R, C] (row-wise: output
    [R][C]; column-wise: output [C][R]) computed chunk by chunk. Returns the
    statistics (and with keep=True the full codes, scales, tensor exponent
    and dequantized values, as oracle.quantize does)."""
    A = OQ.tensor_amax(t32) if amax is None else np.float32(amax)
    R, C = t32.shape
    n_out, k = (R, C) if layout == S.ROWWISE else (C, R)
    step = max(16, (chunk_elems // k) // 16 * 16)
    spans = [(r0, min(n_out, r0 + step)) for r0 in range(0, n_out, step)]

    def one(span):
        ids = np.arange(span[0], span[1])
        if layout == S.ROWWISE:
            return OQ.quantize(t32[span[0]:span[1]], fmt, RND[rounding], seed, tid, amax=A, row_ids=ids)
        return OQ.quantize_colwise(t32, fmt, RND[rounding], seed, tid, amax=A, col_ids=ids)

    parts = list(_pool().map(one, spans))
    st = {"sum_err2": float(sum(p["stats"]["sum_err2"] for p in parts)),
          "sum_x2": float(sum(p["stats"]["sum_x2"] for p in parts)),
          "amax": float(max(p["stats"]["amax"] for p in parts)),
          "n_nonfinite": int(sum(p["stats"]["n_nonfinite"] for p in parts))}
    out = {"stats": st, "texp": parts[0]["texp"], "rows": n_out, "k": k}
    if keep:
        for key in ("packed", "scales", "codes", "xhat", "bad_blocks"):
            if parts[0].get(key) is not None:
                out[key] = np.concatenate([p[key] for p in parts], axis=0)
    return out
