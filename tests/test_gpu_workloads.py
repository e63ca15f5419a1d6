"""GPU parity at the workloads' full sizes, in both launch configurations:
the separate calls (snip_linear_fwd, then snip_linear_bwd reusing the
forward statistics) and the saved-operand calls the benchmark times
(snip_linear_fwd_save, snip_linear_bwd_saved), on every distinct
(layer shape, format) of every workload.

For each layer:
  * the two launch configurations give the same bytes: Y, dX, dW, and the
    saved W^T / X^T operands equal the separate column-wise passes;
  * Y, dX, dW against the oracle's fp64 product of the oracle-quantized
    operands, within 1e-5 * sum|a||b|: every element for the TinyLlama-1B
    block and the 512x512 layer, a seeded sample of rows x columns (tile
    edges included) elsewhere;
  * codes, scales and tensor exponents of all six operands (snip_quantize,
    same tensor ids) bit-exact: whole tensors for the TinyLlama-1B block and
    the 512x512 layer, the sampled rows elsewhere;
  * statistics of all six operands, in both configurations, against the
    whole-tensor oracle (computed in row chunks with the whole tensor's max):
    max|x| and the non-finite count exactly, sum x^2 and sum (Q(x)-x)^2
    within 1e-5.
"""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from oracle import quantize as OQ
from parity import RND, TOL, check_gemm, compare_codes, compare_stats, gpu_codes, oracle_chunked, say

pytestmark = pytest.mark.gpu


def sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    idx.update({0, n - 1})
    for edge in (63, 64, 127, 128, 255, 256):          # tile edges of the 64/128/256 tiles
        if edge < n:
            idx.add(edge)
    return np.array(sorted(idx))


# The six quantized operands of a layer: (name, source, layout, rounding, role).
OPERANDS = (("X", "x", S.ROWWISE, S.RNE, 0), ("W", "w", S.ROWWISE, S.RNE, 1),
            ("dY", "dy", S.ROWWISE, S.SR, 2), ("W^T", "w", S.COLWISE, S.SR, 3),
            ("dY^T", "dy", S.COLWISE, S.SR, 4), ("X^T", "x", S.COLWISE, S.SR, 5))


def run_layer(wl, li, fmt, seed=0, full=False, n_rows=8, n_cols=48, stats=True):
    """full: every output element and every code against the oracle (small
    workloads); otherwise sampled rows x columns. stats: every operand's
    statistics against the whole-tensor oracle."""
    layer = wl.layers[li]
    T, din, dout = wl.tokens, layer.d_in, layer.d_out
    say(f"workload {wl.name} layer {layer.name} ({din}->{dout}, T={T}) fmt={fmt} seed={seed} full={full}")
    x, w, dy = synth.gen_layer(wl, li)
    xd, wd, dyd = x.cuda(), w.cuda(), dy.cuda()
    tid = lambda role: 8 * li + role

    # ---- the separate calls, then the saved-operand calls
    y, st_f = S.linear_fwd(xd, wd, fmt, seed, li)
    dx, dw, st_b = S.linear_bwd(dyd, xd, wd, fmt, fmt, seed, li, fwd_stats=st_f)
    fused = fmt != S.BF16
    if fused:
        y2, saved, st_f4 = S.linear_fwd_save(xd, wd, fmt, seed, li)
        dx2, dw2, st_b2 = S.linear_bwd_saved(dyd, saved, seed, li)
    torch.cuda.synchronize()
    if fused:
        for a, b, n in ((y, y2, "Y"), (dx, dx2, "dX"), (dw, dw2, "dW")):
            assert torch.equal(a, b), f"{wl.name}/{layer.name}: {n} differs between the launch configurations"
        del y2, dx2, dw2

    # ---- quantized operands through snip_quantize (same tensor ids)
    src = {"x": xd, "w": wd, "dy": dyd}
    gq = {}
    if fmt != S.BF16:
        for name, s_, lay, rnd, role in OPERANDS:
            q, _ = S.quantize(src[s_], lay, fmt, rnd, seed, tid(role), with_stats=False)
            gq[name] = q
        torch.cuda.synchronize()
        for name, q in (("W^T", saved.wt), ("X^T", saved.xt)):
            assert torch.equal(q.codes, gq[name].codes), f"{wl.name}/{layer.name}: saved {name} codes"
            if q.scales is not None:
                assert torch.equal(q.scales, gq[name].scales), f"{wl.name}/{layer.name}: saved {name} scales"
            assert torch.equal(q.texp, gq[name].texp), f"{wl.name}/{layer.name}: saved {name} exponent"

    # ---- oracle operands: whole tensors (full) or the sampled rows
    x32, w32, dy32 = (synth.bf16_to_f32(t) for t in (x, w, dy))
    t32 = {"x": x32, "w": w32, "dy": dy32}
    amax = {k: OQ.tensor_amax(v) for k, v in t32.items()}
    rT, rin, rout = (np.arange(T), np.arange(din), np.arange(dout)) if full else (
        sample(T, n_rows, 1000 + li), sample(din, n_cols, 2000 + li), sample(dout, n_cols, 3000 + li))
    sel = {"X": rT, "W": rout, "dY": rT, "W^T": rin, "dY^T": rout, "X^T": rin}
    oq, ostats = {}, {}
    for name, s_, lay, rnd, role in OPERANDS:
        if full or stats:
            o = oracle_chunked(t32[s_], fmt, lay, rnd, seed, tid(role), amax=amax[s_], keep=full)
            ostats[name] = o["stats"]
            if full:
                oq[name] = o
        if not full:
            rows = sel[name]
            if lay == S.ROWWISE:
                oq[name] = OQ.quantize(t32[s_][rows], fmt, RND[rnd], seed, tid(role), amax=amax[s_], row_ids=rows)
            else:
                oq[name] = OQ.quantize_colwise(t32[s_], fmt, RND[rnd], seed, tid(role), amax=amax[s_], col_ids=rows)

    # ---- codes
    for name, q in gq.items():
        compare_codes(gpu_codes(q), oq[name], fmt, rows=None if full else sel[name],
                      what=f"{wl.name}/{layer.name} {name}")
    del gq

    # ---- GEMMs
    def pick(t, r, c):
        return (t if full else t[r][:, c]).cpu().numpy().astype(np.float64)
    check_gemm(pick(y, rT, rout), oq["X"]["xhat"], oq["W"]["xhat"], what=f"{wl.name}/{layer.name} Y")
    check_gemm(pick(dx, rT, rin), oq["dY"]["xhat"], oq["W^T"]["xhat"], what=f"{wl.name}/{layer.name} dX")
    check_gemm(pick(dw, rout, rin), oq["dY^T"]["xhat"], oq["X^T"]["xhat"], what=f"{wl.name}/{layer.name} dW")

    # ---- statistics of both launch configurations
    gsep = dict(zip(["X", "W", "dY", "W^T", "dY^T", "X^T"], S.decode_stats(st_f) + S.decode_stats(st_b)))
    gfus = dict(zip(["X", "W", "W^T", "X^T", "dY", "dY^T"],
                    S.decode_stats(st_f4) + S.decode_stats(st_b2))) if fused else {}
    for name, s_, *_ in OPERANDS:
        for cfg, g in (("separate", gsep), ("saved-operand", gfus)):
            if name not in g:
                continue
            if ostats:
                compare_stats(g[name], ostats[name], what=f"{wl.name}/{layer.name} {cfg} {name}")
            else:
                assert g[name]["amax"] == float(amax[s_]) and g[name]["n_nonfinite"] == 0
    del xd, wd, dyd, y, dx, dw
    torch.cuda.empty_cache()


def layer_index(wl, name):
    return [l.name for l in wl.layers].index(name)


def test_linear512_full():
    wl = synth.WORKLOADS["linear512"]
    run_layer(wl, 0, wl.plan[0], full=True)


@pytest.mark.parametrize("li", range(7))
def test_tinyllama1b_block_full(li):
    """Every layer of the TinyLlama-1B block, in its plan format: every
    output element and every code, in both launch configurations."""
    wl = synth.WORKLOADS["tinyllama1b"]
    run_layer(wl, li, wl.plan[li], full=True)


# Llama-7B: one layer per distinct (shape, format): Q/K 4096->4096 NVFP4,
# V/O 4096->4096 FP8, Gate/Up 4096->11008 NVFP4, Down 11008->4096 NVFP4.
@pytest.mark.parametrize("name", ["Q", "V", "Gate", "Down"])
def test_llama7b_block(name):
    wl = synth.WORKLOADS["llama7b"]
    li = layer_index(wl, name)
    run_layer(wl, li, wl.plan[li])


# Llama-70B (all NVFP4): Q/O 8192->8192, K/V 8192->1024, Gate/Up
# 8192->28672, Down 28672->8192 (K = 28672 in the forward GEMM).
@pytest.mark.parametrize("name", ["Q", "K", "Gate", "Down"])
def test_llama70b_block(name):
    wl = synth.WORKLOADS["llama70b"]
    li = layer_index(wl, name)
    run_layer(wl, li, wl.plan[li])


@pytest.mark.parametrize("fmt", [S.BF16, S.FP8, S.NVFP4, S.MXFP4])
def test_down7b_precision_sweep(fmt):
    """The 7B Down projection at T = 16384 in each format of the sweep (seed
    = format id: the sweep's seeds differ per run)."""
    wl = synth.WORKLOADS["down7b_sweep"]
    run_layer(wl, 0, fmt, seed=fmt)
