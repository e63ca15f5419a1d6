"""GPU parity of the quantized linear layer (forward RTN, backward SR) against
the oracle: every element of Y, dX and dW within 1e-5 * sum|a||b|, the
statistics of each quantized operand within 1e-5, on the 512x512 layer
(T = 256) workload and on ragged shapes in every format combination."""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from oracle import linear as OL
from oracle import quantize as OQ
from parity import RND, TOL, check_gemm, compare_stats, f32, say

pytestmark = pytest.mark.gpu


def run_layer(x, w, dy, fmt_f, fmt_d, fmt_w, seed=0, layer_id=0):
    say(f"linear case T={x.shape[0]} in={x.shape[1]} out={w.shape[0]} fmts=({fmt_f},{fmt_d},{fmt_w}) "
        f"seed={seed} layer={layer_id}")
    xd, wd, dyd = x.cuda(), w.cuda(), dy.cuda()
    y, st_f = S.linear_fwd(xd, wd, fmt_f, seed, layer_id)
    dx, dw, st_b = S.linear_bwd(dyd, xd, wd, fmt_d, fmt_w, seed, layer_id)
    torch.cuda.synchronize()
    x32, w32, dy32 = f32(x), f32(w), f32(dy)
    of = OL.linear_fwd(x32, w32, fmt_f, seed, layer_id)
    ob = OL.linear_bwd(dy32, x32, w32, fmt_d, fmt_w, seed, layer_id)
    check_gemm(y.cpu().numpy().astype(np.float64), of["qx"]["xhat"], of["qw"]["xhat"], what="Y")
    qdy, qwt, qdyt, qxt = ob["q"]
    check_gemm(dx.cpu().numpy().astype(np.float64), qdy["xhat"], qwt["xhat"], what="dX")
    check_gemm(dw.cpu().numpy().astype(np.float64), qdyt["xhat"], qxt["xhat"], what="dW")
    gf = S.decode_stats(st_f)
    gb = S.decode_stats(st_b)
    for i, n in enumerate(["X", "W"]):
        compare_stats(gf[i], of["stats"][i], what=f"fwd stats {n}")
    for i, n in enumerate(["dY", "W^T", "dY^T", "X^T"]):
        compare_stats(gb[i], ob["stats"][i], what=f"bwd stats {n}")
    return y, dx, dw, gf, gb


def test_linear512_workload_nvfp4():
    wl = synth.WORKLOADS["linear512"]
    x, w, dy = synth.gen_layer(wl, 0)
    run_layer(x, w, dy, S.NVFP4, S.NVFP4, S.NVFP4, seed=0, layer_id=0)


@pytest.mark.parametrize("fmts", [(S.FP8, S.FP8, S.FP8), (S.MXFP4, S.MXFP4, S.MXFP4),
                                  (S.BF16, S.BF16, S.BF16), (S.NVFP4, S.FP8, S.NVFP4),
                                  (S.FP8, S.NVFP4, S.MXFP4), (S.BF16, S.NVFP4, S.BF16)])
def test_linear_formats_ragged(fmts):
    T, din, dout = 384, 256, 256
    x = synth.gen_matrix((T, din), seed=1)
    w = synth.gen_matrix((dout, din), seed=2, std=0.02)
    dy = synth.gen_matrix((T, dout), seed=3, std=1e-3)
    run_layer(x, w, dy, *fmts, seed=5, layer_id=3)


def test_linear_ragged_out_and_skips():
    # forward with out not a multiple of the tile; backward with dx only / dw only
    T, din, dout = 256, 384, 144
    x = synth.gen_matrix((T, din), seed=4)
    w = synth.gen_matrix((dout, din), seed=5, std=0.02)
    y, st = S.linear_fwd(x.cuda(), w.cuda(), S.NVFP4, 0, 1)
    torch.cuda.synchronize()
    of = OL.linear_fwd(f32(x), f32(w), S.NVFP4, 0, 1)
    check_gemm(y.cpu().numpy().astype(np.float64), of["qx"]["xhat"], of["qw"]["xhat"], what="Y ragged")
    dout = 256
    w = synth.gen_matrix((dout, din), seed=6, std=0.02)
    dy = synth.gen_matrix((T, dout), seed=7, std=1e-3)
    dx, dw, st = S.linear_bwd(dy.cuda(), x.cuda(), w.cuda(), S.NVFP4, S.NVFP4, 2, 4,
                              need_dx=True, need_dw=False)
    torch.cuda.synchronize()
    assert dw is None
    ob = OL.linear_bwd(f32(dy), f32(x), f32(w), S.NVFP4, S.NVFP4, 2, 4)
    check_gemm(dx.cpu().numpy().astype(np.float64), ob["q"][0]["xhat"], ob["q"][1]["xhat"], what="dX only")
    dx, dw, st = S.linear_bwd(dy.cuda(), x.cuda(), w.cuda(), S.NVFP4, S.NVFP4, 2, 4,
                              need_dx=False, need_dw=True)
    torch.cuda.synchronize()
    assert dx is None
    check_gemm(dw.cpu().numpy().astype(np.float64), ob["q"][2]["xhat"], ob["q"][3]["xhat"], what="dW only")


def test_layer_stats_report():
    wl = synth.WORKLOADS["linear512"]
    x, w, dy = synth.gen_layer(wl, 0)
    _, _, st = S.linear_bwd(dy.cuda(), x.cuda(), w.cuda(), S.NVFP4, S.NVFP4, 0, 0)
    reps, nonfinite = S.layer_stats(st)
    assert not nonfinite
    raw = S.decode_stats(st)
    for r, s in zip(reps, raw):
        assert r["rel_mse"] == pytest.approx(s["sum_err2"] / s["sum_x2"], rel=1e-12)
        assert r["below_sqrt3"] == int(s["sum_x2"] < 3 * s["sum_err2"])
    # NVFP4 noise is well below the gradient norm for Gaussian dY
    assert reps[0]["below_sqrt3"] == 0
    bad = dy.clone()
    bad[0, 0] = float("nan")
    _, _, st = S.linear_bwd(bad.cuda(), x.cuda(), w.cuda(), S.NVFP4, S.NVFP4, 0, 0)
    reps, nonfinite = S.layer_stats(st)
    assert nonfinite and reps[0]["n_nonfinite"] == 1


REPORT_FIELDS = ("rel_mse", "norm_ratio", "below_sqrt3", "amax", "n_nonfinite")


def compare_report(g: dict, o: dict, what: str):
    """One snip_layer_stats record against oracle.linear.report of the
    oracle's statistics of the same tensor: the ratios within the
    statistics' 1e-5 bound (two sums -> 2e-5 on rel-MSE, 1e-5 on the norm
    ratio), the flag, the max and the non-finite count exactly."""
    assert g["below_sqrt3"] == int(o["below_sqrt3"]), f"{what}: sqrt(3) flag {g['below_sqrt3']} vs {o}"
    assert g["rel_mse"] == pytest.approx(o["rel_mse"], rel=2e-5, abs=0), f"{what}: rel_mse"
    if np.isinf(o["norm_ratio"]):
        assert np.isinf(g["norm_ratio"]), f"{what}: norm ratio"
    else:
        assert g["norm_ratio"] == pytest.approx(o["norm_ratio"], rel=1e-5, abs=0), f"{what}: norm ratio"
    assert g["amax"] == np.float32(o["amax"]), f"{what}: amax"
    assert g["n_nonfinite"] == o["n_nonfinite"], f"{what}: non-finite"


def test_layer_stats_matches_oracle_report():
    """snip_layer_stats field by field against oracle.linear.report ["FP4 All
    the Way" summary, Outline: sqrt(3) threshold of gradient norm over
    quantization noise], on a layer's four backward operands and on a
    gradient quantized with stale (delayed-scaling) maxima 2^k above its own:
    the coarser tensor scale pushes the block scales (NVFP4) or the codes
    (FP8) into the subnormal range until the noise exceeds the signal and
    the flag turns on."""
    wl = synth.WORKLOADS["linear512"]
    x, w, dy = synth.gen_layer(wl, 0)
    say("layer_stats vs oracle.report: linear512 backward, NVFP4")
    _, _, st = S.linear_bwd(dy.cuda(), x.cuda(), w.cuda(), S.NVFP4, S.NVFP4, 0, 0)
    reps, nonfinite = S.layer_stats(st)
    assert not nonfinite
    ob = OL.linear_bwd(f32(dy), f32(x), f32(w), S.NVFP4, S.NVFP4, 0, 0)
    for g, o, n in zip(reps, ob["stats"], ("dY", "W^T", "dY^T", "X^T")):
        compare_report(g, OL.report(o), f"linear512 {n}")
    g32 = f32(synth.gen_matrix((256, 512), seed=7, std=1e-3))
    gd = synth.gen_matrix((256, 512), seed=7, std=1e-3).cuda()
    A = float(OQ.tensor_amax(g32))
    flags = set()
    for fmt in (S.NVFP4, S.FP8):
        for rnd in (S.RNE, S.SR):
            for k in (0, 16, 18, 20):
                say(f"layer_stats stale max case fmt={fmt} rounding={rnd} k={k}")
                amax = torch.tensor([np.float32(A * 2.0 ** k)], dtype=torch.float32, device="cuda")
                _, st = S.quantize(gd, S.ROWWISE, fmt, rnd, 5, 11, amax=amax)
                rep, nf = S.layer_stats(st)
                o = OQ.quantize(g32, fmt, RND[rnd], 5, 11, amax=np.float32(A * 2.0 ** k))
                compare_report(rep[0], OL.report(o["stats"]), f"fmt={fmt} rnd={rnd} k={k}")
                flags.add(rep[0]["below_sqrt3"])
    assert flags == {0, 1}, "the cases must cover both sides of the sqrt(3) threshold"


def test_launch_timing_records():
    """snip_timing_*: every launch of a forward + backward is recorded in
    order with its kind, format and algorithmic work, and outputs are the
    same as untimed."""
    wl = synth.WORKLOADS["linear512"]
    x, w, dy = (t.cuda() for t in synth.gen_layer(wl, 0))
    T, din, dout = x.shape[0], x.shape[1], w.shape[0]
    say("timing case linear512 NVFP4")
    y0, _ = S.linear_fwd(x, w, S.NVFP4, 0, 0)
    torch.cuda.synchronize()
    S.timing_start(64)
    y1, st_f = S.linear_fwd(x, w, S.NVFP4, 0, 0)
    S.linear_bwd(dy, x, w, S.NVFP4, S.NVFP4, 0, 0, fwd_stats=st_f)
    recs, untimed = S.timing_read()
    assert untimed == 0
    assert torch.equal(y0, y1)
    kinds = [r["kind"] for r in recs]
    gemms = [r for r in recs if r["kind"] == "gemm"]
    # forward, then the backward's dgrad and wgrad (one grouped launch here)
    assert gemms[0]["work"] == 2.0 * T * din * dout
    assert sum(g["work"] for g in gemms) == 3 * 2.0 * T * din * dout
    assert all(g["format"] == S.NVFP4 for g in gemms)
    assert kinds[0] == "amax" and "quantize" in kinds
    # the layer calls finalise their statistics inside their last GEMM launch
    assert "finalize" not in kinds and kinds[-1] == "gemm"
    q = [r for r in recs if r["kind"] == "quantize"]
    # forward: X, W; backward: dY, W^T, dY^T, X^T (elements read)
    assert sum(r["work"] for r in q) == float(2 * T * din + 2 * dout * din + 2 * T * dout)
    assert all(r["ms"] > 0.0 for r in recs)
    # timing is off again: a further read is an error
    with pytest.raises(S.SnipError):
        S.timing_read()


@pytest.mark.parametrize("fmt", [S.FP8, S.NVFP4])
@pytest.mark.parametrize("shape", [(2176, 1552, 1920, 1664)], ids=["both-128x128"])
def test_bwd_grouped_gemms_match_single_launches(fmt, shape):
    """A layer's dgrad and wgrad GEMMs share one launch when both run unsplit
    on 128x128 tiles (ragged N = in here). Each output must be byte-identical
    to the same GEMM launched alone (dx only, dw only), and the grouped call
    must record a single GEMM launch carrying both GEMMs' flops."""
    T, din, dout, din_saved = shape
    say(f"grouped bwd case T={T} in={din} out={dout} fmt={fmt}")
    x = synth.gen_matrix((T, din), seed=11).cuda()
    w = synth.gen_matrix((dout, din), seed=12, std=0.02).cuda()
    dy = synth.gen_matrix((T, dout), seed=13, std=1e-3).cuda()
    S.timing_start(64)
    dx, dw, _ = S.linear_bwd(dy, x, w, fmt, fmt, 3, 2)
    recs, _ = S.timing_read()
    gemms = [r for r in recs if r["kind"] == "gemm"]
    assert len(gemms) == 1
    assert gemms[0]["work"] == 2.0 * T * din * dout * 2
    assert not [r for r in recs if r["kind"] == "splitk"]
    dx1, _, _ = S.linear_bwd(dy, x, w, fmt, fmt, 3, 2, need_dw=False)
    _, dw1, _ = S.linear_bwd(dy, x, w, fmt, fmt, 3, 2, need_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx1)
    assert torch.equal(dw, dw1)
    # the saved-operand calls (d_in a multiple of 128) take the same grouped
    # launch and give the bytes of the separate calls
    din = din_saved
    x = synth.gen_matrix((T, din), seed=14).cuda()
    w = synth.gen_matrix((dout, din), seed=15, std=0.02).cuda()
    dx, dw, _ = S.linear_bwd(dy, x, w, fmt, fmt, 3, 2)
    y, saved, _ = S.linear_fwd_save(x, w, fmt, 3, 2)
    S.timing_start(64)
    dx2, dw2, _ = S.linear_bwd_saved(dy, saved, 3, 2)
    recs, _ = S.timing_read()
    assert len([r for r in recs if r["kind"] == "gemm"]) == 1
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx) and torch.equal(dw2, dw)
