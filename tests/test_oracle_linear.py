"""Oracle checks (CPU) of the layer compositions: the fused path's oracle
(quantize_dual, linear_fwd_save, linear_bwd_saved) gives exactly what the
separate row-wise / column-wise quantizations and linear_fwd / linear_bwd
give, whose pieces the other oracle tests pin. Also pins the random-stream
roles: the saved W^T and X^T are the dgrad and wgrad B operands."""
import numpy as np
import pytest

import synth
from oracle import linear as OL
from oracle import quantize as OQ

NVFP4, FP8, MXFP4 = 2, 1, 3


def _same_q(a: dict, b: dict):
    for k in ("packed", "scales", "codes", "xhat"):
        if k in a or k in b:
            assert np.array_equal(a[k], b[k]), k
    assert a.get("texp") == b.get("texp")
    assert a["stats"] == b["stats"]


@pytest.mark.parametrize("fmt", [NVFP4, FP8, MXFP4])
def test_saved_path_equals_unfused(fmt):
    T, din, dout = 64, 64, 96
    x = synth.bf16_to_f32(synth.gen_matrix((T, din), seed=1))
    w = synth.bf16_to_f32(synth.gen_matrix((dout, din), seed=2, std=0.02))
    dy = synth.bf16_to_f32(synth.gen_matrix((T, dout), seed=3, std=1e-3))
    f = OL.linear_fwd(x, w, fmt, 7, 3)
    b = OL.linear_bwd(dy, x, w, fmt, fmt, 7, 3)
    fs = OL.linear_fwd_save(x, w, fmt, 7, 3)
    bs = OL.linear_bwd_saved(dy, fs["qwt"], fs["qxt"], fmt, 7, 3)
    assert np.array_equal(fs["y"], f["y"])
    _same_q(fs["qwt"], b["q"][1])
    _same_q(fs["qxt"], b["q"][3])
    assert np.array_equal(bs["dx"], b["dx"])
    assert np.array_equal(bs["dw"], b["dw"])
    _same_q(bs["q"][0], b["q"][0])
    _same_q(bs["q"][1], b["q"][2])


def test_quantize_dual_streams_differ():
    # the two layouts draw from their own tensor ids: swapping them changes
    # the stochastic codes, so a kernel that mixed the streams would fail parity
    x = synth.bf16_to_f32(synth.gen_matrix((64, 64), seed=4))
    r1, c1 = OL.quantize_dual(x, NVFP4, "sr", "sr", 0, 10, 11)
    r2, c2 = OL.quantize_dual(x, NVFP4, "sr", "sr", 0, 11, 10)
    assert not np.array_equal(r1["packed"], r2["packed"])
    assert not np.array_equal(c1["packed"], c2["packed"])
    assert np.array_equal(r1["packed"], OQ.quantize(x, NVFP4, "sr", 0, 10)["packed"])
    assert np.array_equal(c1["packed"], OQ.quantize_colwise(x, NVFP4, "sr", 0, 11)["packed"])
