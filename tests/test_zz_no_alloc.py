"""snip_linear_fwd_save_noalloc (the allocation-free forward: its workspace
is the library's static scratch array) against snip_linear_fwd_save with a
caller workspace, through the C ABI: the same bytes of Y, the saved W^T and
X^T operands and the statistics, on calls in a row that reuse the array
(each later call on a smaller layer than the one before it, so stale
scratch contents from a larger call lie beyond what it writes)."""
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from parity import say

pytestmark = pytest.mark.gpu

CASES = [  # (T, in, out, format, seed): largest first
    (4096, 5632, 2048, S.NVFP4, 3),     # TinyLlama Down, 18.8 MiB of scratch
    (4096, 2048, 2048, S.FP8, 4),       # TinyLlama Q in FP8
    (1024, 512, 768, S.MXFP4, 5),
    (256, 512, 512, S.NVFP4, 6),        # the 512x512 layer
]


def same(a: S.QuantizedTensor, b: S.QuantizedTensor):
    return (torch.equal(a.codes, b.codes) and torch.equal(a.texp, b.texp)
            and (a.scales is None or torch.equal(a.scales, b.scales)))


def test_noalloc_matches_workspace_entry():
    for i, (T, din, dout, fmt, seed) in enumerate(CASES):
        say(f"noalloc case {i}: T={T} in={din} out={dout} fmt={fmt} seed={seed}")
        x = synth.gen_matrix((T, din), seed=10 + i).cuda()
        w = synth.gen_matrix((dout, din), seed=20 + i, std=0.02).cuda()
        y0, sv0, st0 = S.linear_fwd_save(x, w, fmt, seed, i)
        y1, sv1, st1 = S.linear_fwd_save_noalloc(x, w, fmt, seed, i)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), f"case {i}: Y differs"
        assert same(sv0.wt, sv1.wt) and same(sv0.xt, sv1.xt), f"case {i}: saved operands differ"
        assert torch.equal(st0, st1), f"case {i}: statistics differ"


def test_noalloc_rejects_layers_beyond_the_scratch():
    x = torch.empty((8192, 4096), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((11008, 4096), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(S.SnipError) as e:
        S.linear_fwd_save_noalloc(x, w, S.NVFP4, 0, 0)
    assert e.value.code == -5 and "static scratch" in str(e.value)
