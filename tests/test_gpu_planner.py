"""The planner fed by the HIP quantizers' statistics: every statistic of a
small block's operands in FP8 and NVFP4 agrees with the oracle's (1e-5),
and the plan the library's ILP makes from them is optimal for the oracle's
costs (exhaustive search) [SNIP, Abstract: statistics -> divergence
metrics -> integer linear program]."""
import numpy as np
import pytest
import torch

import synth
import sub_byte_mixed_amd as S
from sub_byte_mixed_amd import planner as P
from oracle import planner as OP
from parity import compare_stats, f32, oracle_quant, say

pytestmark = pytest.mark.gpu


def test_plan_from_gpu_statistics():
    shapes = [(256, 256), (256, 512), (512, 256), (256, 256)]
    T = 256
    layers, host = [], []
    for i, (din, dout) in enumerate(shapes):
        x = synth.gen_matrix((T, din), seed=100 + i)
        w = synth.gen_matrix((dout, din), seed=200 + i, std=0.02)
        dy = synth.gen_matrix((T, dout), seed=300 + i, std=1e-3 * (10 ** (i - 1)))
        host.append((x, w, dy))
        layers.append({"x": x.cuda(), "w": w.cuda(), "dy": dy.cuda()})
    formats = [S.FP8, S.NVFP4]
    say("planner statistics case: 4 layers, FP8 and NVFP4")
    stats = P.collect_stats(layers, formats, seed=3)
    torch.cuda.synchronize()
    ostats = []
    for li, (x, w, dy) in enumerate(host):
        per = {}
        for f in formats:
            st = {}
            for t, rr, rc, roles, ids in ((x, S.RNE, S.SR, ("X", "X^T"), (0, 5)),
                                          (w, S.RNE, S.SR, ("W", "W^T"), (1, 3)),
                                          (dy, S.SR, S.SR, ("dY", "dY^T"), (2, 4))):
                orow = oracle_quant(t, S.ROWWISE, f, rr, 3, 8 * li + ids[0])
                ocol = oracle_quant(t, S.COLWISE, f, rc, 3, 8 * li + ids[1])
                st[roles[0]], st[roles[1]] = orow["stats"], ocol["stats"]
                compare_stats(stats[li][f][roles[0]], orow["stats"], what=f"layer {li} fmt {f} {roles[0]}")
                compare_stats(stats[li][f][roles[1]], ocol["stats"], what=f"layer {li} fmt {f} {roles[1]}")
            per[f] = st
        ostats.append(per)
    flops = [3 * 2 * T * a * b for a, b in shapes]
    costs = [P.layer_costs(s) for s in stats]
    plan = P.solve(costs, flops, 0.6, formats, [S.NVFP4])
    name = {S.FP8: "fp8", S.NVFP4: "nvfp4"}
    ocosts = []
    for s in ostats:
        p = OP.proxies({name[f]: v for f, v in s.items()})
        ocosts.append({k: v["forward"] + v["backward"] for k, v in p.items()})
    oplan, ocost = OP.best_plan(ocosts, flops, 0.6)
    mine = sum(ocosts[l][name[plan[l]]] for l in range(len(plan)))
    assert mine == pytest.approx(ocost, rel=1e-5)
    assert sum(fl for fl, p in zip(flops, plan) if p == S.NVFP4) >= 0.6 * sum(flops)
