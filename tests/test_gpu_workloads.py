"""GPU parity at the workloads' full sizes, in both launch configurations:
the saved-operand calls the benchmark times by default (snip_linear_fwd_save,
snip_linear_bwd_saved) and the separate calls (snip_linear_fwd, then
snip_linear_bwd reusing the forward statistics), on sampled outputs the
oracle can compute one by one:

  * Y, dX, dW: a seeded sample of output rows x columns against the oracle's
    fp64 product of the oracle-quantized rows / columns involved (quantized
    with the full-tensor max and their global element indices), within
    1e-5 * sum|a||b|;
  * codes, scales and tensor exponents of every operand (snip_quantize, same
    tensor ids) bit-exact on the sampled rows;
  * statistics: max|x| exactly and sum x^2 within 1e-5 on every tensor;
    sum (Q(x)-x)^2 against the full-tensor oracle where the tensors are small
    enough for it (TinyLlama-1B block, 512x512 layer).
"""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from oracle import quantize as OQ
from parity import TOL, check_gemm, compare_codes, compare_stats, gpu_codes, say

pytestmark = pytest.mark.gpu

RND = {S.RNE: "rne", S.SR: "sr"}


def sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    idx.update({0, n - 1})
    return np.array(sorted(idx))


def oracle_rows(t32, amax, fmt, rnd, seed, tid, rows):
    """Oracle quantization of the given rows of a row-wise operand (amax: the
    whole tensor's max, as the device computes it)."""
    return OQ.quantize(t32[rows], fmt, RND[rnd], seed, tid, amax=amax, row_ids=rows)


def oracle_cols(t32, amax, fmt, rnd, seed, tid, cols):
    """Oracle quantization of the given columns of a column-wise operand
    (rows of the transposed output)."""
    return OQ.quantize_colwise(t32, fmt, RND[rnd], seed, tid, amax=amax, col_ids=cols)


def run_layer(wl, li, fmt, seed=0, full_stats=False, n_rows=8, n_cols=48, fused=False):
    """fused: the saved-operand calls the benchmark times by default
    (snip_linear_fwd_save, snip_linear_bwd_saved: X, W, dY read once)."""
    layer = wl.layers[li]
    T, din, dout = wl.tokens, layer.d_in, layer.d_out
    say(f"workload {wl.name} layer {layer.name} ({din}->{dout}, T={T}) fmt={fmt} seed={seed} fused={fused}")
    x, w, dy = synth.gen_layer(wl, li)
    xd, wd, dyd = x.cuda(), w.cuda(), dy.cuda()
    saved = None
    if fused:
        y, saved, st_f4 = S.linear_fwd_save(xd, wd, fmt, seed, li)
        dx, dw, st_b2 = S.linear_bwd_saved(dyd, saved, seed, li)
        st_f, st_b = st_f4, st_b2
    else:
        y, st_f = S.linear_fwd(xd, wd, fmt, seed, li)
        dx, dw, st_b = S.linear_bwd(dyd, xd, wd, fmt, fmt, seed, li, fwd_stats=st_f)
    torch.cuda.synchronize()
    x32, w32, dy32 = (synth.bf16_to_f32(t) for t in (x, w, dy))
    ax, aw, ady = (OQ.tensor_amax(t) for t in (x32, w32, dy32))

    rT = sample(T, n_rows, 1000 + li)
    rin = sample(din, n_cols, 2000 + li)
    rout = sample(dout, n_cols, 3000 + li)
    tid = lambda role: 8 * li + role
    # forward: Y[rT, rout]
    qx = oracle_rows(x32, ax, fmt, S.RNE, seed, tid(0), rT)
    qw = oracle_rows(w32, aw, fmt, S.RNE, seed, tid(1), rout)
    check_gemm(y[rT][:, rout].cpu().numpy().astype(np.float64), qx["xhat"], qw["xhat"],
               what=f"{wl.name}/{layer.name} Y")
    # dgrad: dX[rT, rin] = Q(dY)[rT] . Q(W^T)[rin]^T
    qdy = oracle_rows(dy32, ady, fmt, S.SR, seed, tid(2), rT)
    qwt = oracle_cols(w32, aw, fmt, S.SR, seed, tid(3), rin)
    check_gemm(dx[rT][:, rin].cpu().numpy().astype(np.float64), qdy["xhat"], qwt["xhat"],
               what=f"{wl.name}/{layer.name} dX")
    # wgrad: dW[rout, rin] = Q(dY^T)[rout] . Q(X^T)[rin]^T
    qdyt = oracle_cols(dy32, ady, fmt, S.SR, seed, tid(4), rout)
    qxt = oracle_cols(x32, ax, fmt, S.SR, seed, tid(5), rin)
    check_gemm(dw[rout][:, rin].cpu().numpy().astype(np.float64), qdyt["xhat"], qxt["xhat"],
               what=f"{wl.name}/{layer.name} dW")

    # codes of every operand on the sampled rows (bf16 has none)
    if saved is not None:                   # the saved backward operands themselves
        compare_codes(gpu_codes(saved.wt), qwt, fmt, rows=rin, what=f"{wl.name}/{layer.name} saved W^T")
        compare_codes(gpu_codes(saved.xt), qxt, fmt, rows=rin, what=f"{wl.name}/{layer.name} saved X^T")
    if fmt != S.BF16 and saved is None:
        for src, lay, rnd, role, rows, o in ((xd, S.ROWWISE, S.RNE, 0, rT, qx), (wd, S.ROWWISE, S.RNE, 1, rout, qw),
                                            (dyd, S.ROWWISE, S.SR, 2, rT, qdy), (wd, S.COLWISE, S.SR, 3, rin, qwt),
                                            (dyd, S.COLWISE, S.SR, 4, rout, qdyt), (xd, S.COLWISE, S.SR, 5, rin, qxt)):
            q, _ = S.quantize(src, lay, fmt, rnd, seed, tid(role), with_stats=False)
            torch.cuda.synchronize()
            compare_codes(gpu_codes(q), o, fmt, rows=rows, what=f"{wl.name}/{layer.name} role {role}")
            del q

    # statistics
    gf, gb = S.decode_stats(st_f), S.decode_stats(st_b)
    tensors = {"X": (x32, ax), "W": (w32, aw), "dY": (dy32, ady)}
    sums = {n: float(np.einsum("ij,ij->", t.astype(np.float64), t.astype(np.float64)))
            for n, (t, _) in tensors.items()}
    names_f, names_b = (["X", "W", "W", "X"], ["dY", "dY"]) if fused else (["X", "W"], ["dY", "W", "dY", "X"])
    for g, n in list(zip(gf, names_f)) + list(zip(gb, names_b)):
        assert g["amax"] == float(tensors[n][1]), f"{n} amax"
        sx2 = sums[n]
        assert abs(g["sum_x2"] - sx2) <= TOL * sx2, f"{n} sum_x2 {g['sum_x2']} vs {sx2}"
        assert g["n_nonfinite"] == 0
    if full_stats and not fused:
        ref = [OQ.quantize(x32, fmt, "rne", seed, tid(0))["stats"],
               OQ.quantize(w32, fmt, "rne", seed, tid(1))["stats"]]
        for g, o, n in zip(gf, ref, names_f):
            compare_stats(g, o, what=f"{wl.name}/{layer.name} fwd {n}")
        ref = [OQ.quantize(dy32, fmt, "sr", seed, tid(2))["stats"],
               OQ.quantize_colwise(w32, fmt, "sr", seed, tid(3))["stats"],
               OQ.quantize_colwise(dy32, fmt, "sr", seed, tid(4))["stats"],
               OQ.quantize_colwise(x32, fmt, "sr", seed, tid(5))["stats"]]
        for g, o, n in zip(gb, ref, ["dY", "W^T", "dY^T", "X^T"]):
            compare_stats(g, o, what=f"{wl.name}/{layer.name} bwd {n}")
    del xd, wd, dyd, y, dx, dw, saved
    torch.cuda.empty_cache()


def test_linear512_full():
    wl = synth.WORKLOADS["linear512"]
    run_layer(wl, 0, wl.plan[0], full_stats=True, n_rows=64, n_cols=128)


@pytest.mark.parametrize("li", range(7))
def test_tinyllama1b_block(li):
    wl = synth.WORKLOADS["tinyllama1b"]
    run_layer(wl, li, wl.plan[li], full_stats=True)


@pytest.mark.parametrize("name", ["Q", "V", "Down"])
def test_llama7b_block(name):
    wl = synth.WORKLOADS["llama7b"]
    li = [l.name for l in wl.layers].index(name)
    run_layer(wl, li, wl.plan[li])


@pytest.mark.parametrize("name", ["K", "Gate"])
def test_llama70b_block(name):
    wl = synth.WORKLOADS["llama70b"]
    li = [l.name for l in wl.layers].index(name)
    run_layer(wl, li, wl.plan[li])


@pytest.mark.parametrize("fmt", [S.BF16, S.FP8, S.NVFP4, S.MXFP4])
def test_down7b_precision_sweep(fmt):
    wl = synth.WORKLOADS["down7b_sweep"]
    run_layer(wl, 0, fmt, seed=fmt)


@pytest.mark.parametrize("li", range(7))
def test_tinyllama1b_block_fused(li):
    """The benchmark's launch configuration: saved-operand calls."""
    wl = synth.WORKLOADS["tinyllama1b"]
    run_layer(wl, li, wl.plan[li], fused=True)


@pytest.mark.parametrize("name", ["V", "Down"])
def test_llama7b_block_fused(name):
    wl = synth.WORKLOADS["llama7b"]
    li = [l.name for l in wl.layers].index(name)
    run_layer(wl, li, wl.plan[li], fused=True)


def test_llama70b_block_fused():
    wl = synth.WORKLOADS["llama70b"]
    li = [l.name for l in wl.layers].index("K")
    run_layer(wl, li, wl.plan[li], fused=True)
