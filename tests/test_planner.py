"""The library's planner (host side): its MILP reaches the exhaustive
optimum of the oracle on random instances, its stats-to-cost step agrees
with the oracle's proxies, and the asynchronous refresh publishes plans."""
import numpy as np
import pytest

import sub_byte_mixed_amd as S
from sub_byte_mixed_amd import planner as P
from oracle import planner as OP

FMT = {S.FP8: "fp8", S.NVFP4: "nvfp4", S.MXFP4: "mxfp4"}


@pytest.mark.parametrize("n_formats", [2, 3])
def test_milp_matches_exhaustive(n_formats):
    rng = np.random.default_rng(n_formats)
    formats = [S.FP8, S.NVFP4, S.MXFP4][:n_formats]
    fp4 = [S.NVFP4, S.MXFP4]
    for trial in range(150):
        L = int(rng.integers(1, 8))
        flops = rng.integers(1, 50, size=L).astype(float)
        costs = [{f: float(rng.exponential()) * (3.0 if f != S.FP8 else 1.0) for f in formats} for _ in range(L)]
        share = float(rng.uniform(0, 1))
        plan = P.solve(costs, flops, share, formats, fp4)
        oplan, ocost = OP.best_plan([{FMT[f]: c[f] for f in formats} for c in costs], list(flops), share,
                                    formats=tuple(FMT[f] for f in formats), fp4=("nvfp4", "mxfp4"))
        if oplan is None:
            assert plan is None
            continue
        cost = sum(costs[l][plan[l]] for l in range(L))
        assert cost == pytest.approx(ocost, rel=1e-9, abs=1e-12)
        assert sum(fl for fl, f in zip(flops, plan) if f in fp4) >= share * flops.sum() * (1 - 1e-9)


def test_costs_match_oracle_proxies():
    rng = np.random.default_rng(1)
    st = {}
    for f in (S.FP8, S.NVFP4):
        st[f] = {r: {"sum_err2": float(rng.uniform(0, 1)), "sum_x2": float(rng.uniform(1, 2))} for r in P.ROLES}
    mine = P.layer_costs(st, lam=1.0)
    ref = OP.proxies(st)
    for f in st:
        assert mine[f] == pytest.approx(ref[f]["forward"] + ref[f]["backward"], rel=1e-15)


def test_async_planner_publishes():
    rng = np.random.default_rng(2)
    flops = [4, 1, 1, 4, 11, 11, 11]
    stats = [{f: {r: {"sum_err2": float(rng.uniform(0.01, 0.02) if f == S.NVFP4 else 1e-4), "sum_x2": 1.0}
                  for r in P.ROLES} for f in (S.FP8, S.NVFP4)} for _ in flops]
    ap = P.AsyncPlanner(flops, 0.8, [S.FP8, S.NVFP4], [S.NVFP4])
    assert ap.plan() is None
    fut = ap.submit(stats)
    plan = fut.result(timeout=30)
    assert ap.plan() == plan and ap.generation == 1
    fp4 = sum(f for f, p in zip(flops, plan) if p == S.NVFP4)
    assert fp4 >= 0.8 * sum(flops)
    ap.close()
