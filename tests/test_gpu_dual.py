"""GPU parity of the fused quantizers (one read of a tensor, both layouts)
and of the saved-operand layer path, against the oracle: codes, block
scales and tensor exponents of both layouts bit-exact, statistics within
1e-5; the layer's Y, dX and dW within 1e-5 * sum|a||b|. The fused path must
also give bit for bit what the separate calls give (same codes, same GEMMs).
Shapes span several 256 x 128 tiles with ragged row and column tails."""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from oracle import linear as OL
from parity import check_gemm, compare_codes, compare_stats, f32, gpu_codes, oracle_quant, say

pytestmark = pytest.mark.gpu

FMTS = [S.NVFP4, S.FP8, S.MXFP4]
ROUNDINGS = [(S.RNE, S.SR), (S.SR, S.SR), (S.RNE, S.RNE), (S.SR, S.RNE)]


def shapes(fmt):
    if fmt == S.MXFP4:
        return [(256, 128), (288, 160), (32, 32), (544, 288), (96, 1056)]
    return [(256, 128), (272, 144), (16, 16), (528, 272), (48, 1040)]


def run_dual(x, fmt, rr, rc, seed=3, tr=7, tc=9, amax=None, xd=None):
    say(f"dual case fmt={fmt} rnd=({rr},{rc}) shape={tuple(x.shape)} seed={seed} amax={amax}")
    if xd is None:
        xd = x.cuda()
    amax_d = None if amax is None else torch.tensor([amax], dtype=torch.float32, device="cuda")
    qr, qc, st = S.quantize_dual(xd, fmt, rr, rc, seed, tr, tc, amax=amax_d)
    torch.cuda.synchronize()
    gs = S.decode_stats(st)
    orow = oracle_quant(x, S.ROWWISE, fmt, rr, seed, tr, amax=amax)
    ocol = oracle_quant(x, S.COLWISE, fmt, rc, seed, tc, amax=amax)
    what = f"fmt={fmt} rnd=({rr},{rc}) shape={tuple(x.shape)}"
    compare_codes(gpu_codes(qr), orow, fmt, what="row-wise " + what)
    compare_codes(gpu_codes(qc), ocol, fmt, what="column-wise " + what)
    fin = orow["stats"]["n_nonfinite"] == 0
    compare_stats(gs[0], orow["stats"], what="row-wise stats " + what, check_err=fin)
    compare_stats(gs[1], ocol["stats"], what="column-wise stats " + what, check_err=fin)
    return qr, qc, gs, orow, ocol


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rounds", ROUNDINGS)
def test_dual_parity(fmt, rounds):
    for i, shp in enumerate(shapes(fmt)):
        x = synth.gen_matrix(shp, seed=40 + i, std=1.0 if i % 2 else 1e-3)
        run_dual(x, fmt, *rounds, seed=11 + i)


@pytest.mark.parametrize("fmt", FMTS)
def test_dual_edge_cases(fmt):
    z = torch.zeros((64, 64), dtype=torch.bfloat16)
    z[::2, 1::3] = -0.0
    _, _, gs, orow, _ = run_dual(z, fmt, S.RNE, S.SR)
    assert orow["stats"]["sum_x2"] == 0.0
    run_dual(torch.full((64, 96), -0.375, dtype=torch.bfloat16), fmt, S.SR, S.SR, seed=9)
    for dist in ("lognormal_mixed", "student_t"):
        run_dual(synth.gen_matrix((96, 256), seed=31, dist=dist), fmt, S.RNE, S.SR, seed=1)
    x = synth.gen_matrix((64, 128), seed=5)
    x[3, 17] = float("nan")
    x[40, 100] = float("inf")
    x[41, 0] = float("-inf")
    _, _, gs, orow, _ = run_dual(x, fmt, S.SR, S.SR, seed=2)
    assert gs[0]["n_nonfinite"] == 3 and gs[1]["n_nonfinite"] == 3


def test_dual_delayed_scaling_and_strided_rows():
    x = synth.gen_x(synth.WORKLOADS["linear512"], 0)         # 0.1 % x20 outliers
    for fmt in (S.NVFP4, S.FP8):
        run_dual(x, fmt, S.RNE, S.SR, seed=4, amax=8.0)      # stale max: saturation
        run_dual(x, fmt, S.SR, S.SR, seed=4, amax=100.0)
    base = synth.gen_matrix((128, 160), seed=8)
    for fmt in FMTS:
        view = base.cuda()[:, :128]                           # ld = 160
        run_dual(base[:, :128].contiguous(), fmt, S.SR, S.RNE, seed=6, xd=view)


@pytest.mark.parametrize("fmt", FMTS)
def test_dual_equals_separate_passes_full_size(fmt):
    """The tinyllama Gate layer's dY (T = 4096, 5632 columns) and W
    (5632 x 2048): the dual pass writes the same bytes as the two separate
    passes, at the size the benchmark runs."""
    wl = synth.WORKLOADS["tinyllama1b"]
    li = [l.name for l in wl.layers].index("Gate")
    for name, t in (("dY", synth.gen_dy(wl, li)), ("W", synth.gen_w(wl, li))):
        say(f"dual vs separate fmt={fmt} tensor={name} shape={tuple(t.shape)}")
        xd = t.cuda()
        qr, qc, st = S.quantize_dual(xd, fmt, S.SR, S.SR, 0, 2, 4)
        ar, sr_ = S.quantize(xd, S.ROWWISE, fmt, S.SR, 0, 2)
        ac, sc_ = S.quantize(xd, S.COLWISE, fmt, S.SR, 0, 4)
        torch.cuda.synchronize()
        for g, a, lay in ((qr, ar, "row"), (qc, ac, "col")):
            assert torch.equal(g.codes, a.codes), f"{name} {lay} codes"
            if g.scales is not None:
                assert torch.equal(g.scales, a.scales), f"{name} {lay} scales"
            assert torch.equal(g.texp, a.texp), f"{name} {lay} exponent"
        # statistics: the dual pass sums a row block in two 8-element fp32
        # halves where the row-wise pass sums 16, so the totals agree to
        # rounding (measured 7e-9 relative), not bit for bit
        d, r, c = S.decode_stats(st), S.decode_stats(sr_)[0], S.decode_stats(sc_)[0]
        for got, ref in ((d[0], r), (d[1], c)):
            assert got["amax"] == ref["amax"] and got["n_nonfinite"] == ref["n_nonfinite"]
            assert got["sum_x2"] == pytest.approx(ref["sum_x2"], rel=1e-6)
            assert got["sum_err2"] == pytest.approx(ref["sum_err2"], rel=1e-6)
        del xd, qr, qc, ar, ac
    torch.cuda.empty_cache()


def run_saved_layer(x, w, dy, fmt, seed=0, layer_id=0):
    say(f"saved layer case T={x.shape[0]} in={x.shape[1]} out={w.shape[0]} fmt={fmt} seed={seed}")
    xd, wd, dyd = x.cuda(), w.cuda(), dy.cuda()
    y, saved, st_f = S.linear_fwd_save(xd, wd, fmt, seed, layer_id)
    dx, dw, st_b = S.linear_bwd_saved(dyd, saved, seed, layer_id)
    # the unfused calls on the same inputs
    y0, st_f0 = S.linear_fwd(xd, wd, fmt, seed, layer_id)
    dx0, dw0, st_b0 = S.linear_bwd(dyd, xd, wd, fmt, fmt, seed, layer_id)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(dx, dx0) and torch.equal(dw, dw0)
    x32, w32, dy32 = f32(x), f32(w), f32(dy)
    of = OL.linear_fwd_save(x32, w32, fmt, seed, layer_id)
    ob = OL.linear_bwd_saved(dy32, of["qwt"], of["qxt"], fmt, seed, layer_id)
    compare_codes(gpu_codes(saved.wt), of["qwt"], fmt, what="saved W^T")
    compare_codes(gpu_codes(saved.xt), of["qxt"], fmt, what="saved X^T")
    check_gemm(y.cpu().numpy().astype(np.float64), of["qx"]["xhat"], of["qw"]["xhat"], what="Y")
    check_gemm(dx.cpu().numpy().astype(np.float64), ob["q"][0]["xhat"], of["qwt"]["xhat"], what="dX")
    check_gemm(dw.cpu().numpy().astype(np.float64), ob["q"][1]["xhat"], of["qxt"]["xhat"], what="dW")
    for g, o, n in zip(S.decode_stats(st_f), of["stats"], ["X", "W", "W^T", "X^T"]):
        compare_stats(g, o, what=f"fwd_save stats {n}")
    for g, o, n in zip(S.decode_stats(st_b), ob["stats"], ["dY", "dY^T"]):
        compare_stats(g, o, what=f"bwd_saved stats {n}")
    return saved


def test_saved_layer_linear512_nvfp4():
    wl = synth.WORKLOADS["linear512"]
    run_saved_layer(*synth.gen_layer(wl, 0), S.NVFP4)


@pytest.mark.parametrize("fmt", FMTS)
def test_saved_layer_formats_ragged(fmt):
    T, din, dout = 384, 256, 640          # 640 columns: a ragged 128-column tile count per 256-row tile
    x = synth.gen_matrix((T, din), seed=1)
    w = synth.gen_matrix((dout, din), seed=2, std=0.02)
    dy = synth.gen_matrix((T, dout), seed=3, std=1e-3)
    run_saved_layer(x, w, dy, fmt, seed=5, layer_id=3)


def test_saved_layer_single_gradient():
    T, din, dout = 256, 384, 256
    x = synth.gen_matrix((T, din), seed=4)
    w = synth.gen_matrix((dout, din), seed=5, std=0.02)
    dy = synth.gen_matrix((T, dout), seed=7, std=1e-3)
    say("saved layer dx only / dw only")
    y, saved, _ = S.linear_fwd_save(x.cuda(), w.cuda(), S.NVFP4, 2, 4)
    dx, dw, st = S.linear_bwd_saved(dy.cuda(), saved, 2, 4, need_dx=True, need_dw=False)
    torch.cuda.synchronize()
    assert dw is None
    dx0, _, st0 = S.linear_bwd(dy.cuda(), x.cuda(), w.cuda(), S.NVFP4, S.NVFP4, 2, 4, need_dw=False)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx0)
    assert S.decode_stats(st)[0]["amax"] == S.decode_stats(st0)[0]["amax"]
    dx, dw, st = S.linear_bwd_saved(dy.cuda(), saved, 2, 4, need_dx=False, need_dw=True)
    _, dw0, _ = S.linear_bwd(dy.cuda(), x.cuda(), w.cuda(), S.NVFP4, S.NVFP4, 2, 4, need_dx=False)
    torch.cuda.synchronize()
    assert dx is None and torch.equal(dw, dw0)


def test_saved_layer_full_size_matches_unfused():
    """Every layer of the tinyllama block at T = 4096 in its planned format:
    the saved-operand path gives bit-identical Y, dX and dW."""
    wl = synth.WORKLOADS["tinyllama1b"]
    for li, (layer, fmt) in enumerate(zip(wl.layers, wl.plan)):
        x, w, dy = (t.cuda() for t in synth.gen_layer(wl, li))
        say(f"saved vs unfused full size layer={layer.name} fmt={fmt} T={x.shape[0]} "
            f"in={x.shape[1]} out={w.shape[0]}")
        y, saved, _ = S.linear_fwd_save(x, w, fmt, 0, li)
        dx, dw, _ = S.linear_bwd_saved(dy, saved, 0, li)
        y0, _ = S.linear_fwd(x, w, fmt, 0, li)
        dx0, dw0, _ = S.linear_bwd(dy, x, w, fmt, fmt, 0, li)
        torch.cuda.synchronize()
        assert torch.equal(y, y0), layer.name
        assert torch.equal(dx, dx0), layer.name
        assert torch.equal(dw, dw0), layer.name
        del x, w, dy, y, saved, dx, dw, y0, dx0, dw0
    torch.cuda.empty_cache()


def _layer_step(xd, wd, dyd, fmt, seed, layer_id, saved, st_f, st_b, amax=(None, None, None)):
    y, _, _ = S.linear_fwd_save(xd, wd, fmt, seed, layer_id, saved=saved, stats=st_f, amax_x=amax[0],
                                amax_w=amax[1])
    dx, dw, _ = S.linear_bwd_saved(dyd, saved, seed, layer_id, stats=st_b, amax_dy=amax[2])
    return y, dx, dw


@pytest.mark.parametrize("fmt", FMTS)
def test_saved_layer_delayed_scaling(fmt):
    """Delayed scaling through the saved-operand calls: the tensor maxima
    come from the previous step's statistics records (read in place, no
    copy), the tensor-max pre-pass is skipped, and the statistics report the
    current tensors' own maxima for the next step.
      step 1: current scaling on (x, w, dy);
      step 2: the same tensors with the maxima of step 1's records -> the
              same bytes as step 1 (the maxima are equal);
      step 3: new tensors (x/2 exactly, 2w, a new dy) with step 2's records,
              which this step overwrites -> the oracle with those stale
              maxima (codes, scales and exponents bit-exact, Y/dX/dW within
              the bound), and statistics of the new tensors (amax = their
              own max)."""
    T, din, dout = 384, 256, 640
    seed, layer_id = 5, 2
    x = synth.gen_matrix((T, din), seed=11)
    w = synth.gen_matrix((dout, din), seed=12, std=0.02)
    dy = synth.gen_matrix((T, dout), seed=13, std=1e-3)
    dev = torch.device("cuda:0")
    say(f"delayed scaling fmt={fmt} T={T} in={din} out={dout}")
    xd, wd, dyd = x.to(dev), w.to(dev), dy.to(dev)
    saved = S.SavedOperands(fmt, T, din, dout, dev)
    st_f, st_b = S.new_stats(4, dev), S.new_stats(2, dev)
    y1, dx1, dw1 = (t.clone() for t in _layer_step(xd, wd, dyd, fmt, seed, layer_id, saved, st_f, st_b))
    torch.cuda.synchronize()
    wt1, xt1 = gpu_codes(saved.wt), gpu_codes(saved.xt)
    sf1, sb1 = st_f.clone(), st_b.clone()

    # step 2: maxima of step 1's records, read from a copy of them
    amax = (S.StatsAmax(sf1, 0), S.StatsAmax(sf1, 1), S.StatsAmax(sb1, 0))
    y2, dx2, dw2 = _layer_step(xd, wd, dyd, fmt, seed, layer_id, saved, st_f, st_b, amax)
    torch.cuda.synchronize()
    assert torch.equal(y2, y1) and torch.equal(dx2, dx1) and torch.equal(dw2, dw1)
    for a, b in ((gpu_codes(saved.wt), wt1), (gpu_codes(saved.xt), xt1)):
        for k in a:
            assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    assert torch.equal(st_f.view(torch.uint8), sf1.view(torch.uint8))
    assert torch.equal(st_b.view(torch.uint8), sb1.view(torch.uint8))

    # step 3: new tensors, maxima read in place from the records this step overwrites
    x3 = (x.float() * 0.5).to(torch.bfloat16)
    w3 = (w.float() * 2.0).to(torch.bfloat16)
    dy3 = synth.gen_matrix((T, dout), seed=14, std=3e-3)
    stale = [S.decode_stats(st_f)[0]["amax"], S.decode_stats(st_f)[1]["amax"], S.decode_stats(st_b)[0]["amax"]]
    amax = (S.StatsAmax(st_f, 0), S.StatsAmax(st_f, 1), S.StatsAmax(st_b, 0))
    y3, dx3, dw3 = _layer_step(x3.to(dev), w3.to(dev), dy3.to(dev), fmt, seed, layer_id, saved, st_f, st_b, amax)
    torch.cuda.synchronize()
    x32, w32, dy32 = f32(x3), f32(w3), f32(dy3)
    of = OL.linear_fwd_save(x32, w32, fmt, seed, layer_id, amax_x=stale[0], amax_w=stale[1])
    ob = OL.linear_bwd_saved(dy32, of["qwt"], of["qxt"], fmt, seed, layer_id, amax_dy=stale[2])
    compare_codes(gpu_codes(saved.wt), of["qwt"], fmt, what="delayed W^T")
    compare_codes(gpu_codes(saved.xt), of["qxt"], fmt, what="delayed X^T")
    check_gemm(y3.cpu().numpy().astype(np.float64), of["qx"]["xhat"], of["qw"]["xhat"], what="delayed Y")
    check_gemm(dx3.cpu().numpy().astype(np.float64), ob["q"][0]["xhat"], of["qwt"]["xhat"], what="delayed dX")
    check_gemm(dw3.cpu().numpy().astype(np.float64), ob["q"][1]["xhat"], of["qxt"]["xhat"], what="delayed dW")
    for g, o, n in zip(S.decode_stats(st_f), of["stats"], ["X", "W", "W^T", "X^T"]):
        compare_stats(g, o, what=f"delayed fwd_save stats {n}")
    for g, o, n in zip(S.decode_stats(st_b), ob["stats"], ["dY", "dY^T"]):
        compare_stats(g, o, what=f"delayed bwd_saved stats {n}")
    # the reported maxima are the new tensors' own (x/2, 2w: exact halving/doubling)
    got = S.decode_stats(st_f)
    assert got[0]["amax"] == stale[0] / 2 and got[1]["amax"] == stale[1] * 2
    assert S.decode_stats(st_b)[0]["amax"] == float(np.max(np.abs(dy32)))
