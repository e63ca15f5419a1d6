"""Pins for the oracle planner (exhaustive search over per-layer formats)
on instances whose optimum is known by hand, and for its stats-derived
proxies on hand-computed statistics. [SNIP, Abstract: an integer linear
program picks per-layer FP8/FP4 formats to minimise the quality loss under
an efficiency target]."""
import math

from oracle import planner as OP


def test_share_zero_takes_each_cheapest():
    costs = [{"fp8": 1.0, "nvfp4": 3.0}, {"fp8": 2.0, "nvfp4": 0.5}, {"fp8": 0.0, "nvfp4": 0.0}]
    plan, cost = OP.best_plan(costs, [1, 1, 1], 0.0)
    assert plan == ["fp8", "nvfp4", "fp8"] and cost == 1.5      # the tie goes to the first format


def test_share_one_forces_fp4():
    costs = [{"fp8": 0.0, "nvfp4": 3.0}] * 4
    plan, cost = OP.best_plan(costs, [5, 6, 7, 8], 1.0)
    assert plan == ["nvfp4"] * 4 and cost == 12.0


def test_knapsack_by_hand():
    # need >= 30 of 60 FP4 FLOPs: {L3} costs 4, {L1, L2} 6, {L2, L3} 5 -> L3 alone
    costs = [{"fp8": 0.0, "nvfp4": 5.0}, {"fp8": 0.0, "nvfp4": 1.0}, {"fp8": 0.0, "nvfp4": 4.0}]
    plan, cost = OP.best_plan(costs, [10, 20, 30], 0.5)
    assert plan == ["fp8", "fp8", "nvfp4"] and cost == 4.0
    # 0.51 needs 30.6: L3 alone no longer suffices -> {L2, L3} at 5
    plan, cost = OP.best_plan(costs, [10, 20, 30], 0.51)
    assert plan == ["fp8", "nvfp4", "nvfp4"] and cost == 5.0


def test_infeasible():
    plan, cost = OP.best_plan([{"fp8": 0.0, "nvfp4": 1.0}], [1], 1.5)
    assert plan is None and math.isinf(cost)


def test_proxies_by_hand():
    st = {"X": {"sum_err2": 1.0, "sum_x2": 100.0}, "W": {"sum_err2": 2.0, "sum_x2": 100.0},
          "dY": {"sum_err2": 3.0, "sum_x2": 100.0}, "W^T": {"sum_err2": 4.0, "sum_x2": 100.0},
          "dY^T": {"sum_err2": 5.0, "sum_x2": 100.0}, "X^T": {"sum_err2": 0.0, "sum_x2": 0.0}}
    p = OP.proxies({"nvfp4": st})["nvfp4"]
    assert abs(p["forward"] - 0.03) < 1e-15 and abs(p["backward"] - 0.12) < 1e-15
