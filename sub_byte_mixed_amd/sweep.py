"""FP4 design-space sweep: the quantization error of every E2M1 format
(block 16 or 32; E4M3, E8M0 or BF16 block scale), under nearest and
stochastic rounding, on the operands a linear layer quantizes, with the
sqrt(3) diagnostic per variant.

"FP4 All the Way" summary, Outline: the study explored block size, scaling
format and rounding and settled on NVFP4 (16 E2M1 values per E4M3 scale),
nearest rounding forward and stochastic rounding in back-propagation and
update; learning suffers once the gradient norm drops below about sqrt(3)
times the quantization noise (read here as ||x|| < sqrt(3) ||Q(x) - x|| of
the same tensor).

Every quantization runs through snip_quantize (the HIP kernels); the sweep
only gathers the statistics and the launch times. Usage:

  python -m sub_byte_mixed_amd.sweep --workload llama7b --layers Gate,Down \
      --out profiles/fp4_design_sweep_llama7b.md

Operand roles per layer: X and W row-wise (forward GEMM), dY row-wise and
W column-wise (dgrad), dY and X column-wise (wgrad).
"""
from __future__ import annotations

import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

ROLES = [("X", "x", 0), ("W", "w", 0), ("dY", "dy", 0), ("W^T", "w", 1), ("dY^T", "dy", 1), ("X^T", "x", 1)]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama7b")
    ap.add_argument("--layers", default="Gate,Down")
    ap.add_argument("--tokens", type=int, default=None, help="rows of X and dY (default: the workload's)")
    ap.add_argument("--reps", type=int, default=5, help="timed launches per pass")
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import torch
    import synth
    import sub_byte_mixed_amd as S

    wl = synth.WORKLOADS[a.workload]
    T = a.tokens or wl.tokens
    names = [l.name for l in wl.layers]
    fmts = [S.NVFP4, S.MXFP4, S.FP4_E4M3_B32, S.FP4_E8M0_B16, S.FP4_BF16_B16, S.FP4_BF16_B32]
    L = S.lib()
    rows = []
    for lname in a.layers.split(","):
        li = names.index(lname)
        t = {"x": synth.gen_x(wl, li, rows=T).cuda(), "w": synth.gen_w(wl, li).cuda(),
             "dy": synth.gen_dy(wl, li, rows=T).cuda()}
        for fmt in fmts:
            blk, kind = S.FP4_LAYOUT[fmt]
            for rnd in (S.RNE, S.SR):
                for role, key, layout in ROLES:
                    x = t[key]
                    q, st = S.quantize(x, layout, fmt, rnd, 0, 8 * li + 2)
                    torch.cuda.synchronize()
                    # device time of the pass's launches (amax, quantize, finalize)
                    S.timing_start(4 * a.reps + 8)
                    for _ in range(a.reps):
                        S.quantize(x, layout, fmt, rnd, 0, 8 * li + 2, out=q, stats=st)
                    recs, _ = S.timing_read()
                    us = sum(r["ms"] for r in recs) / a.reps * 1e3
                    rep, _ = S.layer_stats(st)
                    r = rep[0]
                    n = x.numel()
                    sbytes = L.snip_qtensor_bytes(fmt, q.rows, q.k, 1)
                    rows.append({"layer": lname, "role": role, "format": S.FORMAT_NAMES[fmt], "block": blk,
                                 "scale": kind, "rounding": "sr" if rnd else "rne",
                                 "rel_mse": r["rel_mse"], "norm_ratio": r["norm_ratio"],
                                 "below_sqrt3": r["below_sqrt3"], "us": us,
                                 "gbs": (2 * n + n / 2 + sbytes) / (us * 1e-6) / 1e9})
        del t
        torch.cuda.empty_cache()

    # summary per (format, rounding): mean rel-MSE over the operands, the
    # smallest norm ratio, flags, and the pass rate (amax pre-pass included)
    summ = {}
    for r in rows:
        k = (r["format"], r["block"], r["scale"], r["rounding"])
        s = summ.setdefault(k, {"mse": [], "ratio": [], "flags": 0, "us": 0.0, "bytes": 0.0})
        s["mse"].append(r["rel_mse"])
        s["ratio"].append(r["norm_ratio"])
        s["flags"] += r["below_sqrt3"]
        s["us"] += r["us"]
        s["bytes"] += r["gbs"] * r["us"] * 1e3
    lines = [f"# FP4 design-space sweep on {a.workload} ({a.layers}, T={T})", "",
             "Quantization error of each E2M1 format on the layers' operands (X, W row-wise; dY row-wise;",
             "W^T, dY^T, X^T column-wise), every pass through snip_quantize on the GPU. rel-MSE =",
             "sum (Q(x)-x)^2 / sum x^2; norm ratio = ||x|| / ||Q(x)-x||; a tensor is flagged when the",
             "ratio is below sqrt(3). GB/s: bf16 read + codes + scales written over the pass's device",
             "time (amax, quantize and finalize launches, HIP events). Command (from the repository root):",
             "", "```",
             f"python -m sub_byte_mixed_amd.sweep --workload {a.workload} --layers {a.layers}"
             + (f" --tokens {a.tokens}" if a.tokens else "") + (f" --out {a.out}" if a.out else ""), "```", "",
             "| format | block | scale | rounding | mean rel-MSE | min norm ratio | below sqrt(3) | GB/s |",
             "|---|---|---|---|---|---|---|---|"]
    for (f, b, kd, rd), s in summ.items():
        lines.append(f"| {f} | {b} | {kd} | {rd} | {sum(s['mse']) / len(s['mse']):.5f} | "
                     f"{min(s['ratio']):.2f} | {s['flags']} of {len(s['mse'])} | {s['bytes'] / s['us'] / 1e3:.0f} |")
    lines += ["", "Per operand (rel-MSE, nearest / stochastic):", "",
              "| layer | role | " + " | ".join(S.FORMAT_NAMES[f] for f in fmts) + " |",
              "|---|---|" + "---|" * len(fmts)]
    for lname in a.layers.split(","):
        for role, _, _ in ROLES:
            cells = []
            for f in fmts:
                v = {r["rounding"]: r["rel_mse"] for r in rows
                     if r["layer"] == lname and r["role"] == role and r["format"] == S.FORMAT_NAMES[f]}
                cells.append(f"{v['rne']:.4f} / {v['sr']:.4f}")
            lines.append(f"| {lname} | {role} | " + " | ".join(cells) + " |")
    lines.append("")
    text = "\n".join(lines)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text, flush=True)


if __name__ == "__main__":
    main()
