"""The GPU parity tests quantize large tensors with the oracle in chunks of
output rows, on a thread pool (tests/parity.py `oracle_chunked`). The
chunked result must be the whole-tensor oracle's: every code, scale,
exponent and dequantized value identical, the statistics equal up to fp64
summation order."""
import numpy as np
import pytest

import synth
import sub_byte_mixed_amd as S
from oracle import quantize as OQ
from parity import oracle_chunked


@pytest.mark.parametrize("layout", [S.ROWWISE, S.COLWISE])
@pytest.mark.parametrize("fmt", [S.FP8, S.NVFP4, S.MXFP4, S.BF16])
@pytest.mark.parametrize("rounding", [S.RNE, S.SR])
def test_chunked_oracle_equals_whole_tensor(layout, fmt, rounding):
    x = synth.bf16_to_f32(synth.gen_matrix((352, 640), seed=3, dist="student_t"))
    o = oracle_chunked(x, fmt, layout, rounding, 7, 21, keep=True, chunk_elems=1 << 14)
    rnd = "rne" if rounding == S.RNE else "sr"
    r = OQ.quantize(x, fmt, rnd, 7, 21) if layout == S.ROWWISE else OQ.quantize_colwise(x, fmt, rnd, 7, 21)
    assert o["texp"] == r["texp"] and o["rows"] == r["rows"] and o["k"] == r["k"]
    for key in ("packed", "scales", "codes", "xhat"):
        if r.get(key) is not None:
            assert np.array_equal(o[key], r[key]), key
    for key in ("sum_err2", "sum_x2"):
        assert abs(o["stats"][key] - r["stats"][key]) <= 1e-12 * abs(r["stats"][key])
    assert o["stats"]["amax"] == r["stats"]["amax"]
    assert o["stats"]["n_nonfinite"] == r["stats"]["n_nonfinite"]


def test_chunked_oracle_supplied_max():
    """A supplied max reaches every chunk (delayed scaling)."""
    x = synth.bf16_to_f32(synth.gen_matrix((64, 512), seed=4, std=1e-3))
    A = np.float32(OQ.tensor_amax(x) * 2.0 ** 9)
    o = oracle_chunked(x, S.NVFP4, S.ROWWISE, S.SR, 0, 3, amax=A, keep=True, chunk_elems=1 << 12)
    r = OQ.quantize(x, S.NVFP4, "sr", 0, 3, amax=A)
    assert np.array_equal(o["packed"], r["packed"]) and o["texp"] == r["texp"]
