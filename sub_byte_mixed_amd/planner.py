"""SNIP precision planner: per-layer GEMM formats from quantization
statistics, by an integer linear program with an FP4-FLOP-share target.

[SNIP, Abstract and TL;DR; Fig. 2]: statistics of activations, weights and
gradients are collected periodically; two training-quality metrics, the
forward loss divergence and the backward weight divergence, are estimated
from them; a knapsack-like integer linear program picks each layer's format
(FP8 or FP4) to minimise the total divergence while meeting the efficiency
target (the FP4 share of the GEMM FLOPs); the plan is refreshed
asynchronously while training goes on.

The pages give neither divergence formula. The estimates here are the
statistics the quantize passes already emit: for a layer in format f,
  forward  = sum err^2 / sum x^2 of X plus that of W   (the forward GEMM's
             operands, nearest rounding),
  backward = the same ratio summed over dY, W^T, dY^T and X^T (the two
             backward GEMMs' operands, stochastic rounding),
and the layer's cost is forward + lambda * backward (lambda = 1 unless
given). With statistics measured on the layer's own tensors in every
candidate format, the program is

  minimise   sum_l sum_f cost[l][f] * z[l][f]
  subject to sum_f z[l][f] = 1 for every layer l,
             sum_l flops[l] * z[l][FP4] >= share * sum_l flops[l],
             z binary,

solved by scipy's MILP (HiGHS). Everything on the path that produces the
statistics runs in the HIP kernels (snip_quantize_dual / snip_quantize);
this module is host-side decision logic.
"""
from __future__ import annotations

import threading
from concurrent.futures import Future, ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

ROLES = ("X", "W", "dY", "W^T", "dY^T", "X^T")


def layer_costs(stats_by_format: Dict[int, Dict[str, dict]], lam: float = 1.0) -> Dict[int, float]:
    """cost[f] = forward + lam * backward relative-error proxies of one layer.
    stats_by_format[f][role] holds "sum_err2" and "sum_x2" (snip_stats)."""
    out = {}
    for f, st in stats_by_format.items():
        rel = {r: (st[r]["sum_err2"] / st[r]["sum_x2"] if st[r]["sum_x2"] > 0 else 0.0) for r in ROLES}
        out[f] = (rel["X"] + rel["W"]) + lam * (rel["dY"] + rel["W^T"] + rel["dY^T"] + rel["X^T"])
    return out


def solve(costs: Sequence[Dict[int, float]], flops: Sequence[float], share: float,
          formats: Sequence[int], fp4: Sequence[int]) -> Optional[List[int]]:
    """The ILP above. costs[l][f]; returns a format per layer, or None when
    no plan reaches the share."""
    from scipy.optimize import Bounds, LinearConstraint, milp
    L, F = len(flops), len(formats)
    c = np.array([costs[l][f] for l in range(L) for f in formats], dtype=np.float64)
    one = np.zeros((L, L * F))
    for l in range(L):
        one[l, l * F:(l + 1) * F] = 1.0
    share_row = np.array([[flops[l] if formats[k] in fp4 else 0.0 for l in range(L) for k in range(F)]])
    total = float(sum(flops))
    cons = [LinearConstraint(one, 1.0, 1.0),
            LinearConstraint(share_row, share * total * (1 - 1e-12), np.inf)]
    res = milp(c, constraints=cons, integrality=np.ones(L * F), bounds=Bounds(0, 1))
    if res.status != 0 or res.x is None:
        return None
    z = np.rint(res.x).reshape(L, F)
    return [formats[int(np.argmax(z[l]))] for l in range(L)]


def collect_stats(layers, formats: Sequence[int], seed: int = 0) -> List[Dict[int, Dict[str, dict]]]:
    """Statistics of every layer's six GEMM operands in every candidate
    format, from the HIP quantizers: one dual pass per tensor (X and W:
    row-wise nearest + column-wise stochastic; dY: both stochastic).
    layers: list of dicts with device bf16 tensors "x", "w", "dy"."""
    import sub_byte_mixed_amd as S
    out = []
    for li, d in enumerate(layers):
        per = {}
        for f in formats:
            st = {}
            for key, rr, rc, roles, ids in (("x", S.RNE, S.SR, ("X", "X^T"), (0, 5)),
                                            ("w", S.RNE, S.SR, ("W", "W^T"), (1, 3)),
                                            ("dy", S.SR, S.SR, ("dY", "dY^T"), (2, 4))):
                _, _, s2 = S.quantize_dual(d[key], f, rr, rc, seed, 8 * li + ids[0], 8 * li + ids[1])
                a, b = S.decode_stats(s2)
                st[roles[0]], st[roles[1]] = a, b
            per[f] = st
        out.append(per)
    return out


class AsyncPlanner:
    """Plan refresh off the critical path [SNIP, Fig. 2]: submit() hands the
    latest statistics to a worker thread that solves the ILP; plan() returns
    the newest finished plan (the caller switches formats at a step
    boundary). Submissions are solved one at a time, in order."""

    def __init__(self, flops: Sequence[float], share: float, formats: Sequence[int], fp4: Sequence[int],
                 lam: float = 1.0, initial: Optional[List[int]] = None):
        self.flops, self.share, self.formats, self.fp4, self.lam = list(flops), share, list(formats), list(fp4), lam
        self._plan = initial
        self._lock = threading.Lock()
        self._pool = ThreadPoolExecutor(max_workers=1)
        self._pending: Optional[Future] = None
        self.generation = 0

    def submit(self, stats: List[Dict[int, Dict[str, dict]]]) -> Future:
        costs = [layer_costs(s, self.lam) for s in stats]

        def work():
            p = solve(costs, self.flops, self.share, self.formats, self.fp4)
            with self._lock:
                if p is not None:
                    self._plan = p
                    self.generation += 1
            return p
        with self._lock:
            self._pending = self._pool.submit(work)
            return self._pending

    def plan(self) -> Optional[List[int]]:
        with self._lock:
            return None if self._plan is None else list(self._plan)

    def close(self):
        self._pool.shutdown(wait=True)


def main(argv=None):
    """python -m sub_byte_mixed_amd.planner --workload tinyllama1b --share 0.8
    [--out profiles/snip_plan_tinyllama1b.md]: statistics of every layer's
    operands in FP8 and NVFP4 from the HIP quantizers, the ILP plan, and the
    time of both steps."""
    import argparse
    import os
    import sys
    import time
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="tinyllama1b")
    ap.add_argument("--share", type=float, default=0.8)
    ap.add_argument("--lam", type=float, default=1.0)
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import torch
    import synth
    import sub_byte_mixed_amd as S
    wl = synth.WORKLOADS[a.workload]
    T = wl.tokens
    layers = [dict(zip(("x", "w", "dy"), (t.cuda() for t in synth.gen_layer(wl, li))))
              for li in range(len(wl.layers))]
    flops = [3 * 2 * T * l.d_in * l.d_out for l in wl.layers]
    formats = [S.FP8, S.NVFP4]
    collect_stats(layers[:1], formats)                     # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    stats = collect_stats(layers, formats)
    torch.cuda.synchronize()
    t_collect = time.perf_counter() - t0
    costs = [layer_costs(s, a.lam) for s in stats]
    t0 = time.perf_counter()
    plan = solve(costs, flops, a.share, formats, [S.NVFP4])
    t_solve = time.perf_counter() - t0
    share = sum(f for f, p in zip(flops, plan) if p == S.NVFP4) / sum(flops)
    total = sum(c[p] for c, p in zip(costs, plan))
    lines = [f"# SNIP plan for {a.workload} (T={T}), FP4 FLOP share >= {a.share}", "",
             "Per layer: the stats-derived cost (forward + lambda * backward relative-error proxies, from the",
             "quantize passes' sum err^2 / sum x^2 in each format) and the ILP's choice. Command (from the",
             "repository root):", "", "```",
             f"python -m sub_byte_mixed_amd.planner --workload {a.workload} --share {a.share}"
             + (f" --lam {a.lam}" if a.lam != 1.0 else "") + (f" --out {a.out}" if a.out else ""), "```", "",
             "| layer | d_in -> d_out | GFLOP | cost FP8 | cost NVFP4 | plan |", "|---|---|---|---|---|---|"]
    for l, c, p, fl in zip(wl.layers, costs, plan, flops):
        lines.append(f"| {l.name} | {l.d_in} -> {l.d_out} | {fl / 1e9:.1f} | {c[S.FP8]:.3e} | {c[S.NVFP4]:.3e} | "
                     f"{S.FORMAT_NAMES[p]} |")
    lines += ["", f"FP4 FLOP share {share * 100:.2f} %, total cost {total:.4e}. Statistics of all "
              f"{len(layers)} layers in 2 formats ({len(layers) * 2 * 3} dual quantize passes): "
              f"{t_collect * 1e3:.1f} ms; ILP solve: {t_solve * 1e3:.1f} ms.", ""]
    text = "\n".join(lines)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text, flush=True)


if __name__ == "__main__":
    main()
