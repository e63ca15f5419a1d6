"""Per-configuration performance report of the quantized linear layer.

For each workload (the single 512x512 layer, the TinyLlama-1B, Llama-7B and
Llama-70B blocks, and the 7B Down-projection precision sweep), every layer
runs its forward and backward calls through the library on synthetic inputs
resident in HBM, one layer at a time:

  * the calls are timed whole (HIP events around R repetitions), and
  * the same calls run again with the library's launch timing on, which
    splits each call into its kernels (tensor-max pre-pass, quantize passes,
    the three GEMMs with their split-K sums).

Per GEMM: time, TFLOP/s, fraction of the peak of the MFMA it executes on
(NVFP4 and FP8 are decoded exactly to fp16, so the fp16 peak; MX-FP4 the FP4
peak; BF16 the bf16 peak) and t_roof / t, where t_roof = max(2MNK / peak,
bytes / 8 TB/s) with bytes = both operands' codes and scales once plus the
fp32 output. Per layer: quantize time and credited GB/s (bf16 read + codes
and scales written), the tensor-max pre-passes, the layer's call time and
sum(t_roof) / sum(t). Per block: the same sums and the FP4 share of the GEMM
FLOPs. Every step of the path runs in the HIP kernels; this module only
drives the calls and does the accounting.

  python -m sub_byte_mixed_amd.report [--workloads a,b,...] [--reps R]
                                      [--out profiles/per_config_report.md]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

HBM = 8.0e12
PEAK_FP16 = 2516.6e12                    # MI355X dense fp16/bf16 MFMA
PEAK_FP4 = 10066.3e12                    # dense FP4 MFMA
# credited quantizer bytes per element written by one layout (codes + scales)
OUT_BYTES = {0: 2.0, 1: 1.0, 2: 0.5 + 1 / 16, 3: 0.5 + 1 / 32}
# bytes per operand element a GEMM reads (codes + scales)
GEMM_BYTES = {0: 2.0, 1: 1.0, 2: 0.5 + 1 / 16, 3: 0.5 + 1 / 32}


def exec_peak(fmt: int) -> float:
    return PEAK_FP4 if fmt == 3 else PEAK_FP16


def t_roof_gemm(fmt: int, M: int, N: int, K: int) -> float:
    byts = (M * K + N * K) * GEMM_BYTES[fmt] + 4.0 * M * N
    return max(2.0 * M * N * K / exec_peak(fmt), byts / HBM)


def split_call(recs):
    """One call's launch records -> (gemm seconds in call order, quantize
    seconds, quantize elements by pass, amax seconds, finalize seconds)."""
    gemms, q_s, q_bytes, amax_s, fin_s = [], 0.0, 0.0, 0.0, 0.0
    for r in recs:
        s = r["ms"] * 1e-3
        if r["kind"] == "gemm":
            gemms.append(s)
        elif r["kind"] == "splitk":
            gemms[-1] += s
        elif r["kind"] == "quantize":
            q_s += s
            per = OUT_BYTES[r["format"]] if r["format"] in OUT_BYTES else 2.0
            nlay = 2 if r["layout"] == 2 else 1
            q_bytes += r["work"] * (2.0 + nlay * per)
        elif r["kind"] == "amax":
            amax_s += s
        else:
            fin_s += s
    return gemms, q_s, q_bytes, amax_s, fin_s


def rotation(torch, x, w, dy, min_bytes=512 << 20, most=32):
    """Copies of a layer's inputs that together exceed the 256 MB Infinity
    Cache twice over (at most `most`), so that repeated calls read their
    inputs from HBM as a training step does."""
    per = sum(t.numel() * t.element_size() for t in (x, w, dy))
    n = max(1, min(most, -(-min_bytes // per)))
    return [(x, w, dy)] + [(x.clone(), w.clone(), dy.clone()) for _ in range(n - 1)]


def run_layer(S, torch, dev, wl, li, fmt, inputs, reps, seed=0):
    """Times one layer's forward and backward calls, rotating over the
    copies of its inputs; returns a dict."""
    L = S.lib()
    T, din, dout = wl.tokens, wl.layers[li].d_in, wl.layers[li].d_out
    nrot = len(inputs)
    fused = fmt != S.BF16
    y = torch.empty((T, dout), dtype=torch.float32, device=dev)
    dx = torch.empty((T, din), dtype=torch.float32, device=dev)
    dw = torch.empty((dout, din), dtype=torch.float32, device=dev)
    if fused:
        saved = S.SavedOperands(fmt, T, din, dout, dev)
        st4, st2 = S.new_stats(4, dev), S.new_stats(2, dev)
        wsf = torch.empty(L.snip_linear_fwd_save_workspace(T, din, dout, fmt), dtype=torch.uint8, device=dev)
        wsb = torch.empty(L.snip_linear_bwd_saved_workspace(T, din, dout, fmt), dtype=torch.uint8, device=dev)

        def fwd(r):
            x, w, _ = inputs[r % nrot]
            S.linear_fwd_save(x, w, fmt, seed, li, y=y, saved=saved, stats=st4, ws=wsf)

        def bwd(r):
            S.linear_bwd_saved(inputs[r % nrot][2], saved, seed, li, dx=dx, dw=dw, stats=st2, ws=wsb)
    else:
        stf, stb = S.new_stats(2, dev), S.new_stats(4, dev)
        wsf = torch.empty(L.snip_linear_fwd_workspace(T, din, dout, fmt), dtype=torch.uint8, device=dev)
        wsb = torch.empty(L.snip_linear_bwd_workspace(T, din, dout, fmt, fmt), dtype=torch.uint8, device=dev)

        def fwd(r):
            x, w, _ = inputs[r % nrot]
            S.linear_fwd(x, w, fmt, seed, li, y=y, stats=stf, ws=wsf)

        def bwd(r):
            x, w, dy = inputs[r % nrot]
            S.linear_bwd(dy, x, w, fmt, fmt, seed, li, dx=dx, dw=dw, stats=stb, ws=wsb, fwd_stats=stf)

    out = {"fused": fused, "nrot": nrot}
    for name, call in (("fwd", fwd), ("bwd", bwd)):
        for r in range(2):
            call(r)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            call(r)
        e1.record()
        torch.cuda.synchronize()
        out[name + "_s"] = e0.elapsed_time(e1) * 1e-3 / reps
        S.timing_start(64 * reps)
        for r in range(reps):
            call(r)
        recs, _ = S.timing_read()
        n = len(recs) // reps
        parts = [split_call(recs[i * n:(i + 1) * n]) for i in range(reps)]
        ng = len(parts[0][0])
        out[name + "_gemm_s"] = [sorted(p[0][g] for p in parts)[reps // 2] for g in range(ng)]
        out[name + "_q_s"] = sum(p[1] for p in parts) / reps
        out[name + "_q_bytes"] = parts[0][2]
        out[name + "_amax_s"] = sum(p[3] for p in parts) / reps
    shapes = [(T, dout, din), (T, din, dout), (dout, din, T)]          # fwd, dgrad, wgrad
    out["gemm_s"] = out["fwd_gemm_s"] + out["bwd_gemm_s"]
    out["shapes"] = shapes
    out["flops"] = [2.0 * m * n * k for m, n, k in shapes]
    out["roof_gemm"] = [t_roof_gemm(fmt, *s) for s in shapes]
    out["q_s"] = out["fwd_q_s"] + out["bwd_q_s"]
    out["q_bytes"] = out["fwd_q_bytes"] + out["bwd_q_bytes"]
    out["amax_s"] = out["fwd_amax_s"] + out["bwd_amax_s"]
    out["call_s"] = out["fwd_s"] + out["bwd_s"]
    out["roof"] = sum(out["roof_gemm"]) + out["q_bytes"] / HBM
    return out


def fmt_row(S, name, fmt, r, copy_gbs):
    g = r["gemm_s"]
    def cell(t, fl, rf):
        return f"{t * 1e6:.1f} ({fl / t / 1e12:.0f}, {fl / t / exec_peak(fmt) * 100:.0f} %, {rf / t * 100:.0f} %)"
    fl, rf = r["flops"], r["roof_gemm"]
    if len(g) == 2:
        # dgrad and wgrad ran as one grouped launch: one cell for both
        cells = [cell(g[0], fl[0], rf[0]), "dgrad+wgrad in one launch: " + cell(g[1], fl[1] + fl[2], rf[1] + rf[2]),
                 "(in the dgrad launch)"]
    else:
        cells = [cell(t, f, x) for t, f, x in zip(g, fl, rf)]
    qgbs = r["q_bytes"] / r["q_s"] / 1e9 if r["q_s"] else 0.0
    return (f"| {name} | {S.FORMAT_NAMES[fmt]} | " + " | ".join(cells) +
            f" | {r['q_s'] * 1e6:.1f} ({qgbs:.0f} GB/s, {qgbs * 1e9 / HBM * 100:.0f} %, "
            f"{qgbs / copy_gbs * 100:.0f} %) | {r['amax_s'] * 1e6:.1f} | "
            f"{r['call_s'] * 1e6:.1f} | {r['roof'] / r['call_s'] * 100:.0f} % |")


HEADER = ("| layer | format | fwd GEMM us (TFLOP/s, % peak, t_roof/t) | dgrad GEMM | wgrad GEMM | "
          "quantize us (credited GB/s, % of 8 TB/s, % of copy) | tensor max us | layer fwd+bwd us | "
          "sum t_roof / t |\n"
          "|---|---|---|---|---|---|---|---|---|")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="linear512,tinyllama1b,llama7b,llama70b,down7b_sweep")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import torch
    import synth
    import sub_byte_mixed_amd as S
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    from sub_byte_mixed_amd.profiling import copy_bandwidth
    copy_gbs = copy_bandwidth(torch, dev)
    lines = ["# Per-configuration report: quantized linear layers on one MI355X", "",
             "Each layer's forward and backward calls on synthetic bf16 inputs resident in HBM (saved-operand",
             "calls for FP8/NVFP4/MX-FP4, separate calls for BF16), one layer at a time. Layer time = HIP events",
             f"around {a.reps} repetitions of each call (mean). The kernel split comes from the library's launch",
             "timing (each launch between two HIP events, which adds about 2 us per launch; median over the",
             "repetitions for the GEMMs). GEMM cells: us (TFLOP/s, % of the peak of the MFMA it runs on: fp16",
             "2516.6 TFLOP/s for NVFP4, FP8 and BF16, FP4 10066.3 for MX-FP4; t_roof / t with t_roof =",
             "max(2MNK / peak, operand codes and scales + fp32 output / 8 TB/s)); where a layer's dgrad and",
             "wgrad share one launch, one cell covers both. Quantize = the quantize",
             "passes of both calls, credited with the bf16 read and every layout's codes and scales written,",
             f"against 8 TB/s and against a measured device copy ({copy_gbs:.0f} GB/s read + written, torch copy",
             "of 1 GiB, median of 10). Repetitions rotate over copies of the layer's inputs totalling over 512 MB",
             "(at most 32), so inputs come from HBM as in a training step, not from the 256 MB Infinity Cache.",
             "sum t_roof / t = (the three GEMMs' t_roof + credited quantize bytes / 8 TB/s) over the layer's",
             "call time. Command (from the repository root):", "", "```",
             f"python -m sub_byte_mixed_amd.report --workloads {a.workloads} --reps {a.reps}"
             + (f" --out {a.out}" if a.out else ""), "```", ""]
    for wname in a.workloads.split(","):
        wl = synth.WORKLOADS[wname]
        T = wl.tokens
        sweep = wname == "down7b_sweep"
        runs = []
        if sweep:
            li = 0
            inputs = rotation(torch, *(t.to(dev) for t in synth.gen_layer(wl, li)))
            for fmt in (S.BF16, S.FP8, S.NVFP4, S.MXFP4):
                t0 = time.time()
                r = run_layer(S, torch, dev, wl, li, fmt, inputs, a.reps)
                runs.append((wl.layers[li], fmt, r))
                print(f"[report] {wname} {S.FORMAT_NAMES[fmt]}: {r['call_s'] * 1e3:.3f} ms "
                      f"({time.time() - t0:.1f} s)", flush=True)
            del inputs
        else:
            for li, layer in enumerate(wl.layers):
                t0 = time.time()
                inputs = rotation(torch, *(t.to(dev) for t in synth.gen_layer(wl, li)))
                fmt = wl.plan[li]
                r = run_layer(S, torch, dev, wl, li, fmt, inputs, a.reps)
                runs.append((layer, fmt, r))
                print(f"[report] {wname} {layer.name} {S.FORMAT_NAMES[fmt]}: {r['call_s'] * 1e3:.3f} ms "
                      f"({time.time() - t0:.1f} s)", flush=True)
                del inputs
                torch.cuda.empty_cache()
        lines += [f"## {wname} (T = {T})", "", HEADER]
        for layer, fmt, r in runs:
            lines.append(fmt_row(S, f"{layer.name} {layer.d_in}->{layer.d_out}", fmt, r, copy_gbs))
        if not sweep:
            flops = sum(sum(r["flops"]) for _, _, r in runs)
            fp4 = sum(sum(r["flops"]) for _, f, r in runs if f in (S.NVFP4, S.MXFP4))
            call = sum(r["call_s"] for _, _, r in runs)
            gemm = sum(sum(r["gemm_s"]) for _, _, r in runs)
            roof = sum(r["roof"] for _, _, r in runs)
            q = sum(r["q_s"] for _, _, r in runs)
            qb = sum(r["q_bytes"] for _, _, r in runs)
            am = sum(r["amax_s"] for _, _, r in runs)
            lines += ["", f"Block: {call * 1e3:.3f} ms for {flops / 1e9:.1f} GFLOP of GEMMs "
                      f"({flops / call / 1e12:.0f} TFLOP/s over the layer calls; GEMM kernels alone "
                      f"{flops / gemm / 1e12:.0f} TFLOP/s); quantize {q * 1e3:.3f} ms at {qb / q / 1e9:.0f} GB/s "
                      f"credited; tensor max {am * 1e3:.3f} ms; sum t_roof / t = {roof / call * 100:.0f} %; "
                      f"FP4 share of the GEMM FLOPs {fp4 / flops * 100:.2f} %.", ""]
        else:
            lines.append("")
        del runs
        torch.cuda.empty_cache()
    text = "\n".join(lines)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text, flush=True)


if __name__ == "__main__":
    main()
