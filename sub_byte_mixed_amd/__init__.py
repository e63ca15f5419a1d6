"""sub_byte_mixed_amd -- quantized linear layer (NVFP4 / FP8 / MX-FP4 / BF16)
for AMD MI355X, as a thin Python binding over libsnip's C ABI.

Every step runs in the HIP kernels of libsnip.so; this module only marshals
arguments. PyTorch provides device memory (tensor.data_ptr()) and the stream
(torch.cuda.current_stream().cuda_stream). The functions carry the names of
the C entry points (include/snip.h):

  quantize(x, layout, fmt, rounding, ...)  -> QuantizedTensor, stats
  qgemm(a, b)                              -> fp32 [M, N]
  qgemm_qout(a, b, out_fmt, amax, ...)     -> fp32 [M, N], its row-wise quantization, stats
  linear_fwd(x, w, fmt, ...)               -> y, stats[2]
  linear_bwd(dy, x, w, fmt_d, fmt_w, ...)  -> dx, dw, stats[4]
  quantize_dual(x, fmt, rnd_row, rnd_col, ...)  -> row-wise, column-wise, stats[2]
  linear_fwd_save(x, w, fmt, ...)          -> y, saved (W^T, X^T), stats[4]
  linear_bwd_saved(dy, saved, ...)         -> dx, dw, stats[2]
  layer_stats(stats)                       -> list of per-tensor reports
  timing_start(capacity), timing_read()    -> per-launch kernel times

The library is built in-tree by `python -m sub_byte_mixed_amd.build`. If it is
missing, importing works but every call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsnip.so")

# enums (include/snip.h)
BF16, FP8_E4M3, NVFP4, MXFP4 = 0, 1, 2, 3
FP8 = FP8_E4M3
RNE, SR = 0, 1
ROWWISE, COLWISE, BOTHWISE = 0, 1, 2
# operation codes of snip_workspace_size
(OP_QUANTIZE, OP_QGEMM, OP_LINEAR_FWD, OP_LINEAR_BWD, OP_QUANTIZE_DUAL, OP_LINEAR_FWD_SAVE,
 OP_LINEAR_BWD_SAVED, OP_QGEMM_QOUT) = range(8)
# FP4 design-space variants (quantizer only): E2M1 with another block or scale
FP4_E4M3_B32, FP4_E8M0_B16, FP4_BF16_B16, FP4_BF16_B32 = 4, 5, 6, 7
FORMAT_NAMES = {BF16: "bf16", FP8_E4M3: "fp8_e4m3", NVFP4: "nvfp4", MXFP4: "mxfp4",
                FP4_E4M3_B32: "fp4_e4m3_b32", FP4_E8M0_B16: "fp4_e8m0_b16",
                FP4_BF16_B16: "fp4_bf16_b16", FP4_BF16_B32: "fp4_bf16_b32"}
# (block, scale kind) of every E2M1 format
FP4_LAYOUT = {NVFP4: (16, "e4m3"), MXFP4: (32, "e8m0"), FP4_E4M3_B32: (32, "e4m3"),
              FP4_E8M0_B16: (16, "e8m0"), FP4_BF16_B16: (16, "bf16"), FP4_BF16_B32: (32, "bf16")}
ERRORS = {0: "OK", -1: "NULL", -2: "SHAPE", -3: "ALIGN", -4: "FORMAT", -5: "WORKSPACE",
          -6: "HIP", -7: "NONFINITE"}


class SnipError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libsnip error {code} ({ERRORS.get(code, '?')}): {msg}")
        self.code = code


class QTensorDesc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("k", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_exp", ctypes.c_void_p)]


class TensorReport(ctypes.Structure):
    _fields_ = [("sum_err2", ctypes.c_double), ("sum_x2", ctypes.c_double),
                ("rel_mse", ctypes.c_double), ("norm_ratio", ctypes.c_double),
                ("amax", ctypes.c_float), ("n_nonfinite", ctypes.c_uint32),
                ("below_sqrt3", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class LaunchRecord(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("format", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("work", ctypes.c_double), ("ms", ctypes.c_double)]


LAUNCH_KINDS = {0: "amax", 1: "quantize", 2: "gemm", 3: "splitk", 4: "finalize"}

STATS_BYTES = 24     # sizeof(snip_stats)

_lib = None

_c = ctypes
_SIGS = {
    "snip_quantize": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                 _c.c_int, _c.c_uint64, _c.c_uint32, _c.c_void_p,
                                 _c.POINTER(QTensorDesc), _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                 _c.c_void_p]),
    "snip_qgemm": (_c.c_int, [_c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc), _c.c_void_p,
                              _c.c_int64, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "snip_linear_fwd": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                                   _c.c_int, _c.c_uint64, _c.c_uint32, _c.c_void_p, _c.c_void_p,
                                   _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "snip_linear_bwd": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                                   _c.c_int64, _c.c_int, _c.c_int, _c.c_uint64, _c.c_uint32,
                                   _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                   _c.c_size_t, _c.c_void_p]),
    "snip_quantize_dual": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                      _c.c_int, _c.c_uint64, _c.c_uint32, _c.c_uint32, _c.c_void_p,
                                      _c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc), _c.c_void_p,
                                      _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "snip_linear_fwd_save": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                                        _c.c_int, _c.c_uint64, _c.c_uint32, _c.c_void_p, _c.c_void_p,
                                        _c.c_void_p, _c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc),
                                        _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "snip_linear_fwd_save_noalloc": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                                                _c.c_int, _c.c_uint64, _c.c_uint32, _c.c_void_p, _c.c_void_p,
                                                _c.c_void_p, _c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc),
                                                _c.c_void_p, _c.c_void_p]),
    "snip_linear_bwd_saved": (_c.c_int, [_c.c_void_p, _c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc),
                                         _c.c_int64, _c.c_int64, _c.c_int64, _c.c_uint64, _c.c_uint32,
                                         _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                         _c.c_size_t, _c.c_void_p]),
    "snip_qgemm_qout": (_c.c_int, [_c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc), _c.c_void_p, _c.c_int64,
                                   _c.c_int, _c.c_uint64, _c.c_uint32, _c.c_void_p, _c.POINTER(QTensorDesc),
                                   _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "snip_qgemm_qout_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "snip_layer_stats": (_c.c_int, [_c.c_void_p, _c.c_int, _c.POINTER(TensorReport), _c.c_void_p]),
    "snip_quantize_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "snip_qgemm_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "snip_linear_fwd_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "snip_linear_bwd_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                                _c.c_int]),
    "snip_quantize_dual_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int]),
    "snip_linear_fwd_save_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "snip_linear_bwd_saved_workspace": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "snip_workspace_size": (_c.c_size_t, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "snip_qtensor_bytes": (_c.c_int64, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int]),
    "snip_timing_start": (_c.c_int, [_c.c_int]),
    "snip_timing_read": (_c.c_int, [_c.POINTER(LaunchRecord), _c.c_int, _c.POINTER(_c.c_int64)]),
    "snip_last_error": (_c.c_char_p, []),
    "snip_version": (_c.c_int, []),
}


def lib():
    """The loaded libsnip (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sub_byte_mixed_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(rc: int):
    if rc != 0:
        raise SnipError(rc, lib().snip_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


class StatsAmax:
    """Device address of the amax field of record i of a statistics tensor
    (snip_stats: sum_err2, sum_x2 as fp64, then amax as fp32 at byte 16):
    a supplied tensor max for delayed scaling, read by the kernels without
    a copy. Keeps the statistics tensor alive."""

    def __init__(self, stats: torch.Tensor, i: int):
        if (not stats.is_cuda or stats.dtype != torch.float64 or stats.dim() != 2 or stats.shape[1] != 3
                or not stats.is_contiguous() or not 0 <= i < stats.shape[0]):
            raise ValueError("stats must be a contiguous GPU statistics tensor (new_stats) and i one of its records")
        self.stats, self.i = stats, i

    def data_ptr(self) -> int:
        return self.stats.data_ptr() + STATS_BYTES * self.i + 16


def _amax_ptr(a) -> Optional[int]:
    """None, a device float32 tensor holding max|x|, or a StatsAmax."""
    if a is None:
        return None
    if isinstance(a, StatsAmax):
        return a.data_ptr()
    if not a.is_cuda or a.dtype != torch.float32 or a.numel() < 1:
        raise ValueError("a supplied max must be a device float32 tensor or a StatsAmax")
    return a.data_ptr()


def _require_cuda_bf16(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def new_stats(n: int, device) -> torch.Tensor:
    """Device buffer for n snip_stats records (24 bytes each)."""
    return torch.zeros((n, 3), dtype=torch.float64, device=device)


def decode_stats(stats: torch.Tensor) -> List[dict]:
    """Host decode of snip_stats records (synchronising copy)."""
    raw = stats.detach().cpu().contiguous().numpy().view("u1").reshape(-1, STATS_BYTES)
    out = []
    for r in raw:
        d = r[:16].view("<f8")
        out.append({"sum_err2": float(d[0]), "sum_x2": float(d[1]),
                    "amax": float(r[16:20].view("<f4")[0]),
                    "n_nonfinite": int(r[20:24].view("<u4")[0])})
    return out


class QuantizedTensor:
    """Caller-owned buffers of one quantized operand ([rows][k], K-contiguous)."""

    def __init__(self, fmt: int, rows: int, k: int, device, codes=None, scales=None, texp=None):
        L = lib()
        self.format, self.rows, self.k = fmt, rows, k
        nc = L.snip_qtensor_bytes(fmt, rows, k, 0)
        ns = L.snip_qtensor_bytes(fmt, rows, k, 1)
        if nc < 0:
            raise SnipError(-2, f"invalid quantized tensor shape [{rows}][{k}] for format {fmt}")
        self.codes = codes if codes is not None else torch.empty(nc, dtype=torch.uint8, device=device)
        self.scales = scales if scales is not None else (
            torch.empty(ns, dtype=torch.uint8, device=device) if ns > 0 else None)
        self.texp = texp if texp is not None else torch.zeros(1, dtype=torch.int32, device=device)

    def desc(self) -> QTensorDesc:
        return QTensorDesc(self.format, 0, self.rows, self.k, _ptr(self.codes),
                           _ptr(self.scales), _ptr(self.texp))


def quantize(x: torch.Tensor, layout: int, fmt: int, rounding: int = RNE, seed: int = 0,
             tensor_id: int = 0, amax: Optional[torch.Tensor] = None,
             out: Optional[QuantizedTensor] = None, stats: Optional[torch.Tensor] = None,
             with_stats: bool = True, stream=None) -> Tuple[QuantizedTensor, Optional[torch.Tensor]]:
    """snip_quantize: x bf16 [rows, cols] -> quantized operand ([rows][cols]
    for ROWWISE, [cols][rows] for COLWISE)."""
    _require_cuda_bf16(x, "x")
    L = lib()
    rows, cols = x.shape
    R, K = (rows, cols) if layout == ROWWISE else (cols, rows)
    if out is None:
        out = QuantizedTensor(fmt, R, K, x.device)
    if stats is None and with_stats:
        stats = new_stats(1, x.device)
    ws_n = L.snip_quantize_workspace(rows, cols, layout, fmt)
    ws = _workspace(ws_n, x.device)
    d = out.desc()
    _check(L.snip_quantize(_ptr(x), rows, cols, x.stride(0), layout, fmt, rounding, seed, tensor_id,
                           _ptr(amax), ctypes.byref(d), _ptr(stats), _ptr(ws), ws.numel(),
                           _stream(stream)))
    return out, stats


def qgemm(a: QuantizedTensor, b: QuantizedTensor, out: Optional[torch.Tensor] = None,
          stream=None) -> torch.Tensor:
    """snip_qgemm: fp32 [M, N] = dequant(a) . dequant(b)^T."""
    L = lib()
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=torch.float32, device=a.codes.device)
    da, db = a.desc(), b.desc()
    _check(L.snip_qgemm(ctypes.byref(da), ctypes.byref(db), _ptr(out), out.stride(0), None, 0,
                        _stream(stream)))
    return out


def qgemm_qout(a: QuantizedTensor, b: QuantizedTensor, out_fmt: int, amax, rounding: int = RNE,
               seed: int = 0, tensor_id: int = 0, c: Optional[torch.Tensor] = None,
               q: Optional[QuantizedTensor] = None, stats: Optional[torch.Tensor] = None,
               with_stats: bool = True, stream=None):
    """snip_qgemm_qout: c fp32 [M, N] = dequant(a) . dequant(b)^T and, from
    the same launch, q = c quantized row-wise in out_fmt with the tensor
    scale of the supplied max `amax` (device float32 tensor or StatsAmax).
    Returns (c, q, stats)."""
    L = lib()
    M, N = a.rows, b.rows
    dev = a.codes.device
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32, device=dev)
    if q is None:
        q = QuantizedTensor(out_fmt, M, N, dev)
    if stats is None and with_stats:
        stats = new_stats(1, dev)
    ws = _workspace(L.snip_qgemm_qout_workspace(M, N, a.k, a.format), dev)
    da, db, dq = a.desc(), b.desc(), q.desc()
    _check(L.snip_qgemm_qout(ctypes.byref(da), ctypes.byref(db), _ptr(c), c.stride(0), rounding, seed, tensor_id,
                             _amax_ptr(amax), ctypes.byref(dq), _ptr(stats), _ptr(ws), ws.numel(),
                             _stream(stream)))
    return c, q, stats


def linear_fwd(x: torch.Tensor, w: torch.Tensor, fmt: int, seed: int = 0, layer_id: int = 0,
               y: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
               with_stats: bool = True, ws: Optional[torch.Tensor] = None, stream=None):
    """snip_linear_fwd: y [T, out] fp32 = Q_rne(x) . Q_rne(w)^T."""
    _require_cuda_bf16(x, "x")
    _require_cuda_bf16(w, "w")
    L = lib()
    T, din = x.shape
    dout = w.shape[0]
    if y is None:
        y = torch.empty((T, dout), dtype=torch.float32, device=x.device)
    if stats is None and with_stats:
        stats = new_stats(2, x.device)
    if ws is None:
        ws = _workspace(L.snip_linear_fwd_workspace(T, din, dout, fmt), x.device)
    _check(L.snip_linear_fwd(_ptr(x), _ptr(w), T, din, dout, fmt, seed, layer_id, _ptr(y),
                             _ptr(stats), _ptr(ws), ws.numel(), _stream(stream)))
    return y, stats


def linear_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, fmt_dgrad: int, fmt_wgrad: int,
               seed: int = 0, layer_id: int = 0, need_dx: bool = True, need_dw: bool = True,
               dx: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None,
               stats: Optional[torch.Tensor] = None, with_stats: bool = True,
               ws: Optional[torch.Tensor] = None, fwd_stats: Optional[torch.Tensor] = None,
               stream=None):
    """snip_linear_bwd: dx [T, in] = Q_sr(dy) . Q_sr(w^T)^T, dw [out, in] =
    Q_sr(dy^T) . Q_sr(x^T)^T. fwd_stats: the stats of linear_fwd on the same
    x and w, whose max|x| and max|w| are then reused."""
    for t, n in ((dy, "dy"), (x, "x"), (w, "w")):
        _require_cuda_bf16(t, n)
    L = lib()
    T, dout = dy.shape
    din = x.shape[1]
    if need_dx and dx is None:
        dx = torch.empty((T, din), dtype=torch.float32, device=x.device)
    if need_dw and dw is None:
        dw = torch.empty((dout, din), dtype=torch.float32, device=x.device)
    if stats is None and with_stats:
        stats = new_stats(4, x.device)
    if ws is None:
        ws = _workspace(L.snip_linear_bwd_workspace(T, din, dout, fmt_dgrad, fmt_wgrad), x.device)
    _check(L.snip_linear_bwd(_ptr(dy), _ptr(x), _ptr(w), T, din, dout, fmt_dgrad, fmt_wgrad, seed,
                             layer_id, _ptr(fwd_stats), _ptr(dx) if need_dx else None,
                             _ptr(dw) if need_dw else None, _ptr(stats), _ptr(ws), ws.numel(),
                             _stream(stream)))
    return dx, dw, stats


def quantize_dual(x: torch.Tensor, fmt: int, rounding_row: int = RNE, rounding_col: int = SR,
                  seed: int = 0, tensor_id_row: int = 0, tensor_id_col: int = 1,
                  amax: Optional[torch.Tensor] = None, out_row: Optional[QuantizedTensor] = None,
                  out_col: Optional[QuantizedTensor] = None, stats: Optional[torch.Tensor] = None,
                  with_stats: bool = True, stream=None):
    """snip_quantize_dual: one read of x bf16 [rows, cols] -> (row-wise
    [rows][cols], column-wise [cols][rows], stats[2])."""
    _require_cuda_bf16(x, "x")
    L = lib()
    rows, cols = x.shape
    if out_row is None:
        out_row = QuantizedTensor(fmt, rows, cols, x.device)
    if out_col is None:
        out_col = QuantizedTensor(fmt, cols, rows, x.device)
    if stats is None and with_stats:
        stats = new_stats(2, x.device)
    ws = _workspace(L.snip_quantize_dual_workspace(rows, cols, fmt), x.device)
    dr, dc = out_row.desc(), out_col.desc()
    _check(L.snip_quantize_dual(_ptr(x), rows, cols, x.stride(0), fmt, rounding_row, rounding_col, seed,
                                tensor_id_row, tensor_id_col, _ptr(amax), ctypes.byref(dr), ctypes.byref(dc),
                                _ptr(stats), _ptr(ws), ws.numel(), _stream(stream)))
    return out_row, out_col, stats


class SavedOperands:
    """The backward operands linear_fwd_save writes: W^T [in][out] and
    X^T [in][T], column-wise quantized with stochastic rounding."""

    def __init__(self, fmt: int, T: int, din: int, dout: int, device):
        self.format, self.T, self.din, self.dout = fmt, T, din, dout
        self.wt = QuantizedTensor(fmt, din, dout, device)
        self.xt = QuantizedTensor(fmt, din, T, device)


def linear_fwd_save(x: torch.Tensor, w: torch.Tensor, fmt: int, seed: int = 0, layer_id: int = 0,
                    y: Optional[torch.Tensor] = None, saved: Optional[SavedOperands] = None,
                    stats: Optional[torch.Tensor] = None, with_stats: bool = True,
                    ws: Optional[torch.Tensor] = None, stream=None, amax_x=None, amax_w=None):
    """snip_linear_fwd_save: y = Q_rne(x) . Q_rne(w)^T, plus the backward
    operands W^T and X^T from the same reads. Returns (y, saved, stats[4] =
    {X, W, W^T, X^T}). amax_x, amax_w: supplied tensor maxima (delayed
    scaling: a device float32 tensor or StatsAmax(stats, i) of an earlier
    call's statistics) or None."""
    _require_cuda_bf16(x, "x")
    _require_cuda_bf16(w, "w")
    L = lib()
    T, din = x.shape
    dout = w.shape[0]
    if y is None:
        y = torch.empty((T, dout), dtype=torch.float32, device=x.device)
    if saved is None:
        saved = SavedOperands(fmt, T, din, dout, x.device)
    if stats is None and with_stats:
        stats = new_stats(4, x.device)
    if ws is None:
        ws = _workspace(L.snip_linear_fwd_save_workspace(T, din, dout, fmt), x.device)
    dwt, dxt = saved.wt.desc(), saved.xt.desc()
    _check(L.snip_linear_fwd_save(_ptr(x), _ptr(w), T, din, dout, fmt, seed, layer_id, _amax_ptr(amax_x),
                                  _amax_ptr(amax_w), _ptr(y),
                                  ctypes.byref(dwt), ctypes.byref(dxt), _ptr(stats), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return y, saved, stats


NOALLOC_SCRATCH_BYTES = 32 << 20      # SNIP_NOALLOC_SCRATCH_BYTES


def linear_fwd_save_noalloc(x: torch.Tensor, w: torch.Tensor, fmt: int, seed: int = 0, layer_id: int = 0,
                            y: Optional[torch.Tensor] = None, saved: Optional[SavedOperands] = None,
                            stats: Optional[torch.Tensor] = None, with_stats: bool = True, stream=None,
                            amax_x=None, amax_w=None):
    """snip_linear_fwd_save_noalloc: linear_fwd_save with the library's
    static scratch array as its workspace (the call allocates nothing; the
    outputs y, saved and stats are the caller's). Returns (y, saved, stats)."""
    _require_cuda_bf16(x, "x")
    _require_cuda_bf16(w, "w")
    L = lib()
    T, din = x.shape
    dout = w.shape[0]
    if y is None:
        y = torch.empty((T, dout), dtype=torch.float32, device=x.device)
    if saved is None:
        saved = SavedOperands(fmt, T, din, dout, x.device)
    if stats is None and with_stats:
        stats = new_stats(4, x.device)
    dwt, dxt = saved.wt.desc(), saved.xt.desc()
    _check(L.snip_linear_fwd_save_noalloc(_ptr(x), _ptr(w), T, din, dout, fmt, seed, layer_id, _amax_ptr(amax_x),
                                          _amax_ptr(amax_w), _ptr(y), ctypes.byref(dwt), ctypes.byref(dxt),
                                          _ptr(stats), _stream(stream)))
    return y, saved, stats


def linear_bwd_saved(dy: torch.Tensor, saved: SavedOperands, seed: int = 0, layer_id: int = 0,
                     need_dx: bool = True, need_dw: bool = True, dx: Optional[torch.Tensor] = None,
                     dw: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
                     with_stats: bool = True, ws: Optional[torch.Tensor] = None, stream=None,
                     amax_dy=None):
    """snip_linear_bwd_saved: dY read once (row-wise and column-wise SR),
    dx = Q(dy) . W^T-operand, dw = Q(dy^T) . X^T-operand. Returns (dx, dw,
    stats[2] = {dY, dY^T}). amax_dy: a supplied max for dy, as in
    linear_fwd_save."""
    _require_cuda_bf16(dy, "dy")
    L = lib()
    T, dout = dy.shape
    din = saved.din
    if need_dx and dx is None:
        dx = torch.empty((T, din), dtype=torch.float32, device=dy.device)
    if need_dw and dw is None:
        dw = torch.empty((dout, din), dtype=torch.float32, device=dy.device)
    if stats is None and with_stats:
        stats = new_stats(2, dy.device)
    if ws is None:
        ws = _workspace(L.snip_linear_bwd_saved_workspace(T, din, dout, saved.format), dy.device)
    dwt, dxt = saved.wt.desc(), saved.xt.desc()
    _check(L.snip_linear_bwd_saved(_ptr(dy), ctypes.byref(dwt), ctypes.byref(dxt), T, din, dout, seed,
                                   layer_id, _amax_ptr(amax_dy), _ptr(dx) if need_dx else None, _ptr(dw) if need_dw else None,
                                   _ptr(stats), _ptr(ws), ws.numel(), _stream(stream)))
    return dx, dw, stats


def layer_stats(stats: torch.Tensor, stream=None) -> Tuple[List[dict], bool]:
    """snip_layer_stats: synchronise, copy and derive the per-tensor reports.
    Returns (reports, any_nonfinite)."""
    L = lib()
    n = stats.shape[0]
    arr = (TensorReport * n)()
    rc = L.snip_layer_stats(_ptr(stats), n, arr, _stream(stream))
    if rc not in (0, -7):
        _check(rc)
    reps = [{f: getattr(r, f) for f, _ in TensorReport._fields_ if f != "reserved"} for r in arr]
    return reps, rc == -7


def workspace_bytes(op: str, *args) -> int:
    L = lib()
    return {"quantize": L.snip_quantize_workspace, "qgemm": L.snip_qgemm_workspace,
            "linear_fwd": L.snip_linear_fwd_workspace,
            "linear_bwd": L.snip_linear_bwd_workspace,
            "quantize_dual": L.snip_quantize_dual_workspace,
            "linear_fwd_save": L.snip_linear_fwd_save_workspace,
            "linear_bwd_saved": L.snip_linear_bwd_saved_workspace,
            "qgemm_qout": L.snip_qgemm_qout_workspace}[op](*args)


def version() -> int:
    return lib().snip_version()


def timing_start(capacity: int = 4096) -> None:
    """snip_timing_start: bracket every following kernel launch of the
    library with a pair of HIP events (measurement runs only)."""
    _check(lib().snip_timing_start(int(capacity)))


def timing_read() -> Tuple[List[dict], int]:
    """snip_timing_read: stop timing and return ([{kind, format, layout,
    rounding, work, ms}, ...] in launch order, launches left untimed)."""
    L = lib()
    cap = 1 << 20
    buf = (LaunchRecord * cap)()
    untimed = ctypes.c_int64(0)
    n = L.snip_timing_read(buf, cap, ctypes.byref(untimed))
    if n < 0:
        _check(n)
    recs = [{"kind": LAUNCH_KINDS.get(r.kind, str(r.kind)), "format": r.format, "layout": r.layout,
             "rounding": r.rounding, "work": r.work, "ms": r.ms} for r in buf[:n]]
    return recs, int(untimed.value)
