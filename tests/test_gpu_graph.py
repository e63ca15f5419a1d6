"""The layer calls captured in a HIP graph and replayed give the bytes of the
eager calls.

A caller that replays its training step as a graph (bench.py --graph) must
get every output of every replay equal to the eager result: the library's
launches take all their scratch from the caller's workspace and record no
memset or copy, so a replay is the same kernel sequence on the same
buffers. Each replay runs after eager work that overwrites every output
(fill kernels) and a synchronisation, and is checked in full: y, dx, dw, the
saved W^T / X^T codes, scales and exponents, and the statistics.
Layers of the tinyllama1b block: K (FP8, 64x64 tiles with split-K sums), O
(NVFP4, 128x128 tiles) and Up (NVFP4, 256x128 tiles for the forward GEMM),
through the saved-operand calls and through the separate calls.
"""
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from parity import say

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["tinyllama1b"]


def _layer_buffers(li, fused, dev):
    x, w, dy = (t.to(dev) for t in synth.gen_layer(WL, li))
    fmt = WL.plan[li]
    T, din, dout = WL.tokens, WL.layers[li].d_in, WL.layers[li].d_out
    L = S.lib()
    b = {"x": x, "w": w, "dy": dy, "fmt": fmt,
         "y": torch.empty((T, dout), dtype=torch.float32, device=dev),
         "dx": torch.empty((T, din), dtype=torch.float32, device=dev),
         "dw": torch.empty((dout, din), dtype=torch.float32, device=dev)}
    if fused:
        b["saved"] = S.SavedOperands(fmt, T, din, dout, dev)
        b["st_f"], b["st_b"] = S.new_stats(4, dev), S.new_stats(2, dev)
        b["ws_f"] = torch.empty(L.snip_linear_fwd_save_workspace(T, din, dout, fmt), dtype=torch.uint8, device=dev)
        b["ws_b"] = torch.empty(L.snip_linear_bwd_saved_workspace(T, din, dout, fmt), dtype=torch.uint8, device=dev)
    else:
        b["st_f"], b["st_b"] = S.new_stats(2, dev), S.new_stats(4, dev)
        b["ws_f"] = torch.empty(L.snip_linear_fwd_workspace(T, din, dout, fmt), dtype=torch.uint8, device=dev)
        b["ws_b"] = torch.empty(L.snip_linear_bwd_workspace(T, din, dout, fmt, fmt), dtype=torch.uint8,
                                device=dev)
    return b


def _step(b, li, fused):
    if fused:
        S.linear_fwd_save(b["x"], b["w"], b["fmt"], 0, li, y=b["y"], saved=b["saved"], stats=b["st_f"],
                          ws=b["ws_f"])
        S.linear_bwd_saved(b["dy"], b["saved"], 0, li, dx=b["dx"], dw=b["dw"], stats=b["st_b"], ws=b["ws_b"])
    else:
        S.linear_fwd(b["x"], b["w"], b["fmt"], 0, li, y=b["y"], stats=b["st_f"], ws=b["ws_f"])
        S.linear_bwd(b["dy"], b["x"], b["w"], b["fmt"], b["fmt"], 0, li, dx=b["dx"], dw=b["dw"],
                     stats=b["st_b"], ws=b["ws_b"], fwd_stats=b["st_f"])


def _outputs(b, fused):
    out = {"y": b["y"], "dx": b["dx"], "dw": b["dw"], "st_f": b["st_f"], "st_b": b["st_b"]}
    if fused:
        for name, q in (("wt", b["saved"].wt), ("xt", b["saved"].xt)):
            out[name + ".codes"] = q.codes
            if q.scales is not None:
                out[name + ".scales"] = q.scales
            out[name + ".texp"] = q.texp
    return out


def _same_bytes(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _clobber(outs):
    for t in outs.values():
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(0x5A if t.dtype == torch.uint8 else -77)


@pytest.mark.parametrize("fused", [True, False], ids=["saved", "separate"])
@pytest.mark.parametrize("li", [1, 3, 5], ids=["K_fp8", "O_nvfp4", "Up_nvfp4"])
def test_layer_graph_replay_matches_eager(li, fused):
    dev = torch.device("cuda:0")
    say(f"graph replay layer={WL.layers[li].name} fmt={WL.plan[li]} fused={fused}")
    b = _layer_buffers(li, fused, dev)
    _step(b, li, fused)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in _outputs(b, fused).items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(b, li, fused)                                # warm-up on the capture side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(b, li, fused)
    torch.cuda.synchronize()

    outs = _outputs(b, fused)
    for rep in range(3):
        _clobber(outs)                                     # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert _same_bytes(v, ref[k]), f"replay {rep}: {k} differs from the eager result"
    # and eager calls after the replays still agree
    _clobber(outs)
    _step(b, li, fused)
    torch.cuda.synchronize()
    for k, v in outs.items():
        assert _same_bytes(v, ref[k]), f"eager after replays: {k} differs"
    del g
