"""C-ABI checks that need no GPU: the library loads, exports every function
include/snip.h declares, sizes buffers, and rejects bad arguments with the
documented status codes before any HIP call (so these calls are safe on a
machine without a GPU: the fake device addresses below are never touched)."""
import ctypes
import os
import re

import pytest

import sub_byte_mixed_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "snip.h")

# fake, 256-byte-aligned device addresses: validation must reject before use
P = 0x7F0000000000
P2 = P + 0x100000
P3 = P + 0x200000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(S.LIB_PATH):
        from sub_byte_mixed_amd import build
        build.build()
    return S.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(snip_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 24
    for n in names:
        assert hasattr(L, n), n
    # and nothing else is exported under the snip_ prefix
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r"\bT (snip_[a-z0-9_]+)", out)))
    assert exported == names


def test_version_and_sizes(L):
    assert L.snip_version() == 100
    assert L.snip_qtensor_bytes(S.NVFP4, 4, 32, 0) == 64
    assert L.snip_qtensor_bytes(S.NVFP4, 4, 32, 1) == 8
    assert L.snip_qtensor_bytes(S.MXFP4, 4, 64, 1) == 8
    assert L.snip_qtensor_bytes(S.FP8, 4, 32, 0) == 128
    assert L.snip_qtensor_bytes(S.FP8, 4, 32, 1) == 0
    assert L.snip_qtensor_bytes(S.BF16, 4, 32, 0) == 256
    assert L.snip_qtensor_bytes(S.MXFP4, 4, 48, 0) == -1       # k % 32
    assert L.snip_qtensor_bytes(9, 4, 32, 0) == -1
    assert L.snip_quantize_workspace(16, 16, S.ROWWISE, S.NVFP4) > 0
    assert L.snip_quantize_workspace(0, 16, S.ROWWISE, S.NVFP4) == 0
    f = L.snip_linear_fwd_workspace(256, 512, 512, S.NVFP4)
    # quantized X and W: codes + scales at least
    assert f >= 256 * 512 // 2 + 256 * 512 // 16 + 512 * 512 // 2 + 512 * 512 // 16
    b = L.snip_linear_bwd_workspace(256, 512, 512, S.NVFP4, S.FP8)
    assert b >= 2 * (256 * 512 // 2) + 2 * 256 * 512
    assert L.snip_linear_bwd_workspace(256, 512, 512, 7, S.FP8) == 0


def qdesc(fmt, rows, k, codes=P2, scales=P3, texp=P3 + 0x1000):
    return S.QTensorDesc(fmt, 0, rows, k, codes, scales, texp)


def err(L):
    return L.snip_last_error().decode()


def quant(L, x=P, rows=64, cols=64, ld=64, layout=0, fmt=S.NVFP4, rnd=0, out=None, ws=P + 0x400000,
          ws_bytes=1 << 20, amax=None, stats=None):
    if out is None:
        R, K = (rows, cols) if layout == 0 else (cols, rows)
        out = qdesc(fmt, R, K)
    return L.snip_quantize(x, rows, cols, ld, layout, fmt, rnd, 0, 0, amax, ctypes.byref(out), stats,
                           ws, ws_bytes, None)


def test_quantize_validation(L):
    assert quant(L, x=None) == -1 and "x is NULL" in err(L)
    assert quant(L, fmt=9) == -4
    assert quant(L, rnd=3) == -4
    assert quant(L, layout=2) == -4
    assert quant(L, cols=40, ld=40) == -2                       # cols % 16
    assert quant(L, ld=60) == -2                                # ld < cols
    assert quant(L, rows=0) == -2
    assert quant(L, layout=1, rows=40) == -2                    # K = rows % 16
    assert quant(L, fmt=S.MXFP4, cols=48, ld=48) == -2          # MX K % 32
    assert quant(L, out=qdesc(S.FP8, 64, 64)) == -4             # format mismatch
    assert quant(L, out=qdesc(S.NVFP4, 64, 32)) == -2           # shape mismatch
    assert quant(L, layout=1, rows=64, cols=32, ld=32, out=qdesc(S.NVFP4, 64, 32)) == -2
    assert quant(L, out=qdesc(S.NVFP4, 64, 64, scales=None)) == -1
    assert quant(L, out=qdesc(S.NVFP4, 64, 64, texp=None)) == -1
    assert quant(L, x=P + 2) == -3
    assert quant(L, out=qdesc(S.NVFP4, 64, 64, codes=P2 + 8)) == -3
    assert quant(L, ws=None) == -5
    assert quant(L, ws_bytes=1024) == -5 and "workspace" in err(L)


def test_qgemm_validation(L):
    a, b = qdesc(S.NVFP4, 64, 256), qdesc(S.NVFP4, 32, 256)
    c = P + 0x800000
    assert L.snip_qgemm(None, ctypes.byref(b), c, 32, None, 0, None) == -1
    assert L.snip_qgemm(ctypes.byref(a), ctypes.byref(b), None, 32, None, 0, None) == -1
    b8 = qdesc(S.FP8, 32, 256, scales=None)
    assert L.snip_qgemm(ctypes.byref(a), ctypes.byref(b8), c, 32, None, 0, None) == -4
    bk = qdesc(S.NVFP4, 32, 128)
    assert L.snip_qgemm(ctypes.byref(a), ctypes.byref(bk), c, 32, None, 0, None) == -2
    a96, b96 = qdesc(S.NVFP4, 64, 96), qdesc(S.NVFP4, 32, 96)
    assert L.snip_qgemm(ctypes.byref(a96), ctypes.byref(b96), c, 32, None, 0, None) == -2
    assert L.snip_qgemm(ctypes.byref(a), ctypes.byref(b), c, 16, None, 0, None) == -2   # ldc < N
    assert L.snip_qgemm(ctypes.byref(a), ctypes.byref(b), c + 4, 32, None, 0, None) == -3
    bad = qdesc(5, 32, 256)
    assert L.snip_qgemm(ctypes.byref(a), ctypes.byref(bad), c, 32, None, 0, None) == -4
    # operands of 4 GiB of codes or more are refused before any HIP call
    # (the GEMM kernels address rows with 32-bit byte offsets)
    a8, big8 = qdesc(S.FP8, 64, 4096, scales=None), qdesc(S.FP8, 1 << 20, 4096, scales=None)
    assert L.snip_qgemm(ctypes.byref(a8), ctypes.byref(big8), c, 1 << 20, None, 0, None) == -2
    assert "4 GiB" in err(L)
    a4, bigf4 = qdesc(S.NVFP4, 64, 4096), qdesc(S.NVFP4, 1 << 21, 4096)   # 4 GiB of nibbles
    assert L.snip_qgemm(ctypes.byref(a4), ctypes.byref(bigf4), c, 1 << 21, None, 0, None) == -2


def test_linear_validation(L):
    ws, y = P + 0x1000000, P + 0x2000000
    assert L.snip_linear_fwd(None, P2, 64, 128, 64, S.NVFP4, 0, 0, y, None, ws, 1 << 30, None) == -1
    assert L.snip_linear_fwd(P, P2, 64, 96, 64, S.NVFP4, 0, 0, y, None, ws, 1 << 30, None) == -2
    assert L.snip_linear_fwd(P, P2, 64, 128, 64, 11, 0, 0, y, None, ws, 1 << 30, None) == -4
    assert L.snip_linear_fwd(P, P2, 64, 128, 64, S.NVFP4, 0, 0, y, None, ws, 100, None) == -5
    assert L.snip_linear_fwd(P, P2 + 1, 64, 128, 64, S.NVFP4, 0, 0, y, None, ws, 1 << 30, None) == -3
    # backward: dgrad needs out % 128, wgrad needs T % 128
    dx, dw = P + 0x3000000, P + 0x4000000
    assert L.snip_linear_bwd(P, P2, P3, 128, 64, 96, S.NVFP4, S.NVFP4, 0, 0, None, dx, None, None, ws,
                             1 << 30, None) == -2
    assert L.snip_linear_bwd(P, P2, P3, 96, 64, 128, S.NVFP4, S.NVFP4, 0, 0, None, None, dw, None, ws,
                             1 << 30, None) == -2
    assert L.snip_linear_bwd(P, None, P3, 128, 64, 128, S.NVFP4, S.NVFP4, 0, 0, None, dx, dw, None, ws,
                             1 << 30, None) == -1
    assert L.snip_linear_bwd(P, P2, P3, 128, 64, 128, S.NVFP4, 9, 0, 0, None, dx, dw, None, ws,
                             1 << 30, None) == -4
    assert L.snip_linear_bwd(P, P2, P3, 128, 64, 128, S.NVFP4, S.FP8, 0, 0, None, dx, dw, None, ws,
                             64, None) == -5
    # a GEMM operand of 4 GiB of codes: X [2^20][4096] in FP8 (forward A),
    # X^T [4096][2^20] (wgrad B)
    big = 1 << 20
    assert L.snip_linear_fwd(P, P2, big, 4096, 128, S.FP8, 0, 0, y, None, ws, 1 << 30, None) == -2
    assert "4 GiB" in err(L)
    assert L.snip_linear_bwd(P, P2, P3, big, 4096, 128, S.FP8, S.FP8, 0, 0, None, None, dw, None, ws,
                             1 << 30, None) == -2


def dual(L, x=P, rows=64, cols=64, ld=64, fmt=S.NVFP4, rr=0, rc=1, out_row=None, out_col=None,
         ws=P + 0x400000, ws_bytes=1 << 20, amax=None, stats=None):
    out_row = out_row or qdesc(fmt, rows, cols)
    out_col = out_col or qdesc(fmt, cols, rows, codes=P2 + 0x10000)
    return L.snip_quantize_dual(x, rows, cols, ld, fmt, rr, rc, 0, 0, 1, amax, ctypes.byref(out_row),
                                ctypes.byref(out_col), stats, ws, ws_bytes, None)


def test_quantize_dual_validation(L):
    assert dual(L, x=None) == -1
    assert dual(L, fmt=S.BF16) == -4 and "not NVFP4" in err(L)
    assert dual(L, rr=2) == -4
    assert dual(L, rc=-1) == -4
    assert dual(L, rows=40) == -2                               # rows % 16
    assert dual(L, cols=40, ld=40) == -2                        # cols % 16
    assert dual(L, fmt=S.MXFP4, rows=48) == -2                  # MX: % 32
    assert dual(L, ld=60) == -2
    assert dual(L, out_row=qdesc(S.NVFP4, 64, 32)) == -2        # shape mismatch
    assert dual(L, out_col=qdesc(S.FP8, 64, 64, scales=None)) == -4
    assert dual(L, out_col=qdesc(S.NVFP4, 64, 64, texp=None)) == -1
    assert dual(L, x=P + 2) == -3
    assert dual(L, ws_bytes=1024) == -5 and "workspace" in err(L)
    assert L.snip_quantize_dual_workspace(64, 64, S.NVFP4) > 0
    assert L.snip_quantize_dual_workspace(64, 64, S.BF16) == 0


def test_saved_linear_validation(L):
    ws, y, dx, dw = P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000
    T, din, dout = 256, 128, 384
    wt, xt = qdesc(S.NVFP4, din, dout), qdesc(S.NVFP4, din, T, codes=P2 + 0x20000)
    big = 1 << 30

    def fwd(x=P, w=P2, T=T, din=din, dout=dout, fmt=S.NVFP4, wt=wt, xt=xt, ws_bytes=big, amax_x=None, amax_w=None):
        return L.snip_linear_fwd_save(x, w, T, din, dout, fmt, 0, 0, amax_x, amax_w, y, ctypes.byref(wt),
                                      ctypes.byref(xt), None, ws, ws_bytes, None)
    assert fwd(x=None) == -1
    assert fwd(fmt=S.BF16) == -4
    assert fwd(T=200) == -2                                      # T % 128
    assert fwd(dout=200, wt=qdesc(S.NVFP4, din, 200)) == -2
    assert fwd(wt=qdesc(S.NVFP4, din, 256)) == -2                # wt shape
    assert fwd(xt=qdesc(S.FP8, din, T, scales=None)) == -4       # xt format
    assert fwd(x=P + 4) == -3
    assert fwd(amax_x=P + 2) == -3                               # supplied max: 4-byte aligned
    assert fwd(amax_w=P + 6) == -3
    assert fwd(T=1 << 20, din=4096, dout=128, fmt=S.FP8) == -2 and "4 GiB" in err(L)   # X^T: 4 GiB of codes
    assert fwd(ws_bytes=64) == -5
    assert L.snip_linear_fwd_save_workspace(T, din, dout, S.NVFP4) > 0

    def bwd(dy=P, T=T, din=din, dout=dout, wt=wt, xt=xt, dx=dx, dw=dw, ws_bytes=big, amax_dy=None):
        return L.snip_linear_bwd_saved(dy, ctypes.byref(wt), ctypes.byref(xt), T, din, dout, 0, 0, amax_dy, dx,
                                       dw, None, ws, ws_bytes, None)
    assert bwd(dy=None) == -1
    assert bwd(xt=qdesc(S.MXFP4, din, T)) == -4                  # formats differ
    assert bwd(wt=qdesc(S.BF16, din, dout)) == -4
    assert bwd(T=128) == -2                                      # xt is [in][256]
    assert bwd(dout=200) == -2
    assert bwd(dx=dx + 4) == -3
    assert bwd(amax_dy=P + 1) == -3
    assert bwd(ws_bytes=64) == -5
    assert L.snip_linear_bwd_saved_workspace(T, din, dout, S.BF16) == 0


def test_fp4_variant_sizes_and_rejections(L):
    assert L.snip_qtensor_bytes(S.FP4_E4M3_B32, 4, 64, 0) == 128
    assert L.snip_qtensor_bytes(S.FP4_E4M3_B32, 4, 64, 1) == 8
    assert L.snip_qtensor_bytes(S.FP4_E8M0_B16, 4, 64, 1) == 16
    assert L.snip_qtensor_bytes(S.FP4_BF16_B16, 4, 64, 1) == 32     # 2-byte scales
    assert L.snip_qtensor_bytes(S.FP4_BF16_B32, 4, 64, 1) == 16
    assert L.snip_qtensor_bytes(S.FP4_BF16_B32, 4, 48, 0) == -1     # k % 32
    assert L.snip_qtensor_bytes(8, 4, 64, 0) == -1
    assert quant(L, fmt=S.FP4_E4M3_B32, cols=48, ld=48) == -2        # K % 32
    assert quant(L, fmt=S.FP4_BF16_B16, layout=1, rows=40) == -2     # K = rows % 16
    a, b = qdesc(S.FP4_BF16_B16, 64, 256), qdesc(S.FP4_BF16_B16, 32, 256)
    assert L.snip_qgemm(ctypes.byref(a), ctypes.byref(b), P + 0x800000, 32, None, 0, None) == -4
    assert "quantizer-only" in err(L)
    ws, y = P + 0x1000000, P + 0x2000000
    assert L.snip_linear_fwd(P, P2, 64, 128, 64, S.FP4_E8M0_B16, 0, 0, y, None, ws, 1 << 30, None) == -4
    assert L.snip_qgemm_workspace(64, 64, 128, S.FP4_E4M3_B32) == 0


def test_layer_stats_validation(L):
    rep = (S.TensorReport * 2)()
    assert L.snip_layer_stats(None, 2, rep, None) == -1
    assert L.snip_layer_stats(P, 0, rep, None) == -2
    assert L.snip_layer_stats(P, 2, None, None) == -1


def test_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros((16, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        S.quantize(x, S.ROWWISE, S.NVFP4)


def test_supplied_max_arguments_are_checked():
    """Delayed-scaling maxima are checked in the binding before any library
    call: a StatsAmax needs a contiguous GPU statistics tensor and a record
    index inside it, a plain supplied max a device float32 tensor."""
    import torch
    with pytest.raises(ValueError):
        S.StatsAmax(torch.zeros((2, 3), dtype=torch.float64), 0)       # not on the GPU
    with pytest.raises(ValueError):
        S._amax_ptr(torch.zeros(1, dtype=torch.float32))                # not on the GPU
    assert S._amax_ptr(None) is None


def test_timing_argument_errors(L):
    assert L.snip_timing_start(0) == -2
    assert L.snip_timing_start((1 << 20) + 1) == -2
    n = ctypes.c_int64(-1)
    assert L.snip_timing_read(None, 0, ctypes.byref(n)) == -4     # not started
    assert "not started" in err(L)


def test_workspace_size_matches_per_call_sizers(L):
    """snip_workspace_size(op, M, N, K, format) is each call's own sizer."""
    for fmt in (S.BF16, S.FP8, S.NVFP4, S.MXFP4):
        for (T, din, dout) in ((256, 512, 512), (4096, 2048, 256), (4096, 8192, 28672), (240, 2048, 2000)):
            assert L.snip_workspace_size(S.OP_QUANTIZE, T, din, 0, fmt) == \
                L.snip_quantize_workspace(T, din, S.ROWWISE, fmt)
            assert L.snip_workspace_size(S.OP_QGEMM, T, dout, din, fmt) == L.snip_qgemm_workspace(T, dout, din, fmt)
            assert L.snip_workspace_size(S.OP_LINEAR_FWD, T, dout, din, fmt) == \
                L.snip_linear_fwd_workspace(T, din, dout, fmt)
            assert L.snip_workspace_size(S.OP_LINEAR_BWD, T, dout, din, fmt) == \
                L.snip_linear_bwd_workspace(T, din, dout, fmt, fmt)
            assert L.snip_workspace_size(S.OP_QUANTIZE_DUAL, T, din, 0, fmt) == \
                L.snip_quantize_dual_workspace(T, din, fmt)
            assert L.snip_workspace_size(S.OP_LINEAR_FWD_SAVE, T, dout, din, fmt) == \
                L.snip_linear_fwd_save_workspace(T, din, dout, fmt)
            assert L.snip_workspace_size(S.OP_LINEAR_BWD_SAVED, T, dout, din, fmt) == \
                L.snip_linear_bwd_saved_workspace(T, din, dout, fmt)
            assert L.snip_workspace_size(S.OP_QGEMM_QOUT, T, dout, din, fmt) == \
                L.snip_qgemm_qout_workspace(T, dout, din, fmt)
    # a split-K plan needs scratch: the skinny K projection's wgrad
    assert L.snip_workspace_size(S.OP_QGEMM, 256, 2048, 4096, S.FP8) > 0
    assert L.snip_workspace_size(S.OP_LINEAR_FWD, 256, 512, 512, S.NVFP4) > 0
    assert L.snip_workspace_size(8, 256, 512, 512, S.NVFP4) == 0
    assert L.snip_workspace_size(-1, 256, 512, 512, S.NVFP4) == 0
    assert L.snip_workspace_size(S.OP_QGEMM, 0, 512, 512, S.NVFP4) == 0


def test_noalloc_validates_before_any_hip_call(L):
    """The allocation-free forward checks every argument, the size of the
    static scratch included, before its first HIP call (fake device
    addresses below are never touched)."""
    d_wt = S.QTensorDesc(S.NVFP4, 0, 4096, 11008, P2, P3, P3 + 4096)
    d_xt = S.QTensorDesc(S.NVFP4, 0, 4096, 8192, P2, P3, P3 + 4096)
    rc = L.snip_linear_fwd_save_noalloc(P, P, 8192, 4096, 11008, S.NVFP4, 0, 0, None, None, P,
                                        ctypes.byref(d_wt), ctypes.byref(d_xt), None, None)
    assert rc == -5
    assert b"static scratch" in L.snip_last_error()
    assert L.snip_linear_fwd_save_workspace(8192, 4096, 11008, S.NVFP4) > S.NOALLOC_SCRATCH_BYTES
    rc = L.snip_linear_fwd_save_noalloc(P, None, 256, 512, 512, S.NVFP4, 0, 0, None, None, P,
                                        ctypes.byref(d_wt), ctypes.byref(d_xt), None, None)
    assert rc == -1
    rc = L.snip_linear_fwd_save_noalloc(P, P, 256, 500, 512, S.NVFP4, 0, 0, None, None, P,
                                        ctypes.byref(d_wt), ctypes.byref(d_xt), None, None)
    assert rc == -2
    rc = L.snip_linear_fwd_save_noalloc(P, P, 256, 512, 512, S.BF16, 0, 0, None, None, P,
                                        ctypes.byref(d_wt), ctypes.byref(d_xt), None, None)
    assert rc == -4
