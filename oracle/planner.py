"""Precision plan by exhaustive search (test infrastructure; the library's
planner must reach the same optimum).

[SNIP, Abstract and TL;DR]: per-layer formats (FP8 or FP4) are chosen by an
integer linear program that minimises the total quality loss (the layers'
forward loss divergence and backward weight divergence) while the FP4 share
of the GEMM FLOPs meets a target; the program is knapsack-like.

Definition used here: every layer l takes one format f from `formats`;
cost(plan) = sum_l c[l][f_l]; feasible iff the FLOPs of the layers in FP4
reach `share` of all FLOPs. The optimum is the least cost over all
feasible plans, found by trying every plan (len(formats)^L of them), so
only small L are meant. Ties: the first optimal plan in lexicographic
order of the format indices.
"""
from __future__ import annotations

import itertools


def best_plan(costs, flops, share: float, formats=("fp8", "nvfp4"), fp4=("nvfp4",)):
    """costs: list (per layer) of dict format -> cost; flops: list of layer
    FLOPs. Returns (plan as a list of formats, cost), or (None, inf) when no
    plan reaches the share."""
    total = float(sum(flops))
    best, best_cost = None, float("inf")
    for choice in itertools.product(range(len(formats)), repeat=len(flops)):
        fp4_flops = sum(fl for fl, c in zip(flops, choice) if formats[c] in fp4)
        if fp4_flops < share * total - 1e-9 * total:
            continue
        cost = sum(costs[l][formats[c]] for l, c in enumerate(choice))
        if cost < best_cost:
            best, best_cost = [formats[c] for c in choice], cost
    return best, best_cost


def proxies(stats_by_format: dict) -> dict:
    """Stats-derived divergence proxies of one layer for each candidate
    format: forward = rel-MSE(X) + rel-MSE(W); backward = rel-MSE of the four
    backward operands (dY, W^T, dY^T, X^T). stats_by_format[f] is a dict
    role -> {"sum_err2", "sum_x2"} with roles X, W, dY, W^T, dY^T, X^T."""
    out = {}
    for f, st in stats_by_format.items():
        rel = {r: (s["sum_err2"] / s["sum_x2"] if s["sum_x2"] > 0 else 0.0) for r, s in st.items()}
        out[f] = {"forward": rel["X"] + rel["W"],
                  "backward": rel["dY"] + rel["W^T"] + rel["dY^T"] + rel["X^T"]}
    return out
