"""Benchmark: one step = forward + backward of every linear layer (Q, K, V, O,
Gate, Up, Down) of a Llama-like block through the quantized linear layer
(quantize X/W with round-to-nearest, GEMM; quantize dY/W/dY/X with Philox
stochastic rounding, dgrad and wgrad GEMMs; per-tensor statistics), on
synthetic bf16 inputs already resident in HBM.

By default each layer runs the saved-operand path (snip_linear_fwd_save /
snip_linear_bwd_saved): X, W and dY are each read once by a dual quantizer
that writes both of their layouts; the results are bit-identical to the
separate calls (--path unfused), which read X and W again in the backward
pass and dY twice.

Prints one JSON line: whole-step GEMM throughput (TFLOP/s over the step's
wall time, quantizers and statistics included), the dominant kernel against
its MFMA roofline, the quantizers' credited HBM bandwidth, and the CPU
oracle timed on a bounded sample on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--path fused|unfused] [--scaling current|delayed]
                       [--no-cpu-baseline] [--graph]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {  # MI355X published dense peaks
    "hbm_gbs": 8000.0,
    "fp16_tflops": 2516.6, "bf16_tflops": 2516.6, "fp8_tflops": 5033.2, "fp4_tflops": 10066.3,
}
METRIC = "qGEMM TFLOP/s (FP4/FP8) + quantize GB/s per Llama layer fwd+bwd, % of roofline"
# credited quantizer bytes per element (bf16 read + codes + scales written)
QBYTES = {1: 2 + 1.0, 2: 2 + 0.5 + 1 / 16, 3: 2 + 0.5 + 1 / 32, 0: 2 + 2.0}
# a dual pass reads once and writes both layouts
QBYTES_DUAL = {f: 2 + 2 * (b - 2) for f, b in QBYTES.items()}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b",
                    help="llama70b (the largest single-GPU block, default), llama7b, tinyllama1b, ...")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None, help="output rows per quantize pass of the oracle sample")
    ap.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    ap.add_argument("--path", choices=("fused", "unfused"), default="fused",
                    help="fused: one read of X, W and dY per step (saved-operand calls)")
    ap.add_argument("--scaling", choices=("current", "delayed"), default="current",
                    help="delayed: tensor maxima from the previous step's statistics (fused path only; "
                         "the first warm-up step uses current scaling)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU: the quantized linear layer is "
                                   "measured on a single MI355X; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import synth
    import sub_byte_mixed_amd as S

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]
    T = wl.tokens
    seed = 0
    L = S.lib()

    # ---------------------------------------------------------------- inputs
    fused = args.path == "fused" and all(f != S.BF16 for f in wl.plan)
    layers = []
    for li, layer in enumerate(wl.layers):
        x, w, dy = synth.gen_layer(wl, li)
        fmt = wl.plan[li]
        d = {
            "name": layer.name, "fmt": fmt, "din": layer.d_in, "dout": layer.d_out,
            "x": x.to(dev), "w": w.to(dev), "dy": dy.to(dev),
            "y": torch.empty((T, layer.d_out), dtype=torch.float32, device=dev),
            "dx": torch.empty((T, layer.d_in), dtype=torch.float32, device=dev),
            "dw": torch.empty((layer.d_out, layer.d_in), dtype=torch.float32, device=dev),
            "st_f": S.new_stats(2, dev), "st_b": S.new_stats(4, dev),
        }
        d["ws_f"] = torch.empty(L.snip_linear_fwd_workspace(T, layer.d_in, layer.d_out, fmt),
                                dtype=torch.uint8, device=dev)
        d["ws_b"] = torch.empty(L.snip_linear_bwd_workspace(T, layer.d_in, layer.d_out, fmt, fmt),
                                dtype=torch.uint8, device=dev)
        if fused:
            d["saved"] = S.SavedOperands(fmt, T, layer.d_in, layer.d_out, dev)
            d["st_f4"], d["st_b2"] = S.new_stats(4, dev), S.new_stats(2, dev)
            d["ws_fs"] = torch.empty(L.snip_linear_fwd_save_workspace(T, layer.d_in, layer.d_out, fmt),
                                     dtype=torch.uint8, device=dev)
            d["ws_bs"] = torch.empty(L.snip_linear_bwd_saved_workspace(T, layer.d_in, layer.d_out, fmt),
                                     dtype=torch.uint8, device=dev)
        layers.append(d)
    torch.cuda.synchronize()

    delayed = {"on": False}
    if args.scaling == "delayed" and not fused:
        print(json.dumps({"error": "--scaling delayed needs the fused path and no BF16 layer"}))
        sys.exit(2)

    def step_fused():
        for li, d in enumerate(layers):
            # delayed scaling: the maxima are read in place from the records the
            # step overwrites, i.e. the previous step's statistics
            am = ((S.StatsAmax(d["st_f4"], 0), S.StatsAmax(d["st_f4"], 1), S.StatsAmax(d["st_b2"], 0))
                  if delayed["on"] else (None, None, None))
            S.linear_fwd_save(d["x"], d["w"], d["fmt"], seed, li, y=d["y"], saved=d["saved"], stats=d["st_f4"],
                              ws=d["ws_fs"], amax_x=am[0], amax_w=am[1])
            S.linear_bwd_saved(d["dy"], d["saved"], seed, li, dx=d["dx"], dw=d["dw"], stats=d["st_b2"],
                               ws=d["ws_bs"], amax_dy=am[2])

    def step_unfused():
        for li, d in enumerate(layers):
            S.linear_fwd(d["x"], d["w"], d["fmt"], seed, li, y=d["y"], stats=d["st_f"], ws=d["ws_f"])
            S.linear_bwd(d["dy"], d["x"], d["w"], d["fmt"], d["fmt"], seed, li, dx=d["dx"], dw=d["dw"],
                         stats=d["st_b"], ws=d["ws_b"], fwd_stats=d["st_f"])

    step = step_fused if fused else step_unfused
    gemm_flops = sum(3 * 2 * T * d["din"] * d["dout"] for d in layers)

    if args.scaling == "delayed":
        step()                                   # current scaling: seeds every statistics record
        torch.cuda.synchronize()
        delayed["on"] = True
    graph = None
    if args.graph:
        step()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    run = graph.replay if graph is not None else step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        run()
        ev[i + 1].record()                       # per-step boundaries (percentiles)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = max(ev[0].elapsed_time(ev[-1]), wall * 1e3) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    pct = {f"p{q}": round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)}
    from sub_byte_mixed_amd.profiling import copy_bandwidth
    copy_gbs = copy_bandwidth(torch, dev)
    value = gemm_flops / (ms_step * 1e-3) / 1e12

    # ---------------------------------------------------- per-kernel timing
    # The same steps again, eagerly, with every kernel launch of the library
    # bracketed by HIP events on the stream it is launched on.
    S.timing_start(len(layers) * 40 * args.steps + 64)
    for _ in range(args.steps):
        step()
    recs, untimed = S.timing_read()
    if untimed:
        raise RuntimeError(f"{untimed} launches were not timed")
    gemm_by_fmt = {}
    quant = {"bytes": 0.0, "ms": 0.0, "launches": 0}
    other_ms = {}
    by_class = {}
    for r in recs:
        if r["kind"] in ("quantize", "amax"):
            fname = S.FORMAT_NAMES.get(r["format"], "any")
            rn = {0: "rne", 1: "sr"}
            if r["kind"] == "amax":
                key, nb = "amax", 2.0 * r["work"]
            elif r["layout"] == S.BOTHWISE:     # rounding = row + 2 * column
                key = f"quantize {fname} dual row-{rn[r['rounding'] & 1]} col-{rn[r['rounding'] >> 1]}"
                nb = r["work"] * QBYTES_DUAL[r["format"]]
            else:
                key = f"quantize {fname} {'row' if r['layout'] == 0 else 'col'} {rn[r['rounding']]}"
                nb = r["work"] * QBYTES[r["format"]]
            c = by_class.setdefault(key, {"ms": 0.0, "bytes": 0.0, "launches": 0, "elems": 0.0,
                                          "dual": (fname, rn[r["rounding"] & 1].upper(), rn[r["rounding"] >> 1].upper())
                                          if r["kind"] == "quantize" and r["layout"] == S.BOTHWISE else None})
            c["ms"] += r["ms"]
            c["bytes"] += nb
            c["launches"] += 1
            c["elems"] += r["work"]
        if r["kind"] == "gemm":
            g = gemm_by_fmt.setdefault(r["format"], {"ms": 0.0, "flops": 0.0, "launches": 0})
            g["ms"] += r["ms"]
            g["flops"] += r["work"]
            g["launches"] += 1
        elif r["kind"] == "quantize":
            quant["ms"] += r["ms"]
            quant["bytes"] += r["work"] * (QBYTES_DUAL if r["layout"] == S.BOTHWISE else QBYTES)[r["format"]]
            quant["launches"] += 1
        else:
            other_ms[r["kind"]] = other_ms.get(r["kind"], 0.0) + r["ms"]
    dom_fmt = max(gemm_by_fmt, key=lambda f: gemm_by_fmt[f]["ms"])
    # algorithmic HBM bytes of the dominant format's GEMMs: both operands'
    # codes and scales read once, the fp32 product written once
    ebytes = {S.BF16: 2.0, S.FP8: 1.0, S.NVFP4: 0.5 + 1 / 16, S.MXFP4: 0.5 + 1 / 32}[dom_fmt]
    shapes = [(T, d["dout"], d["din"]) for d in layers if d["fmt"] == dom_fmt]
    shapes = [s_ for (t, o, i) in shapes for s_ in ((t, o, i), (t, i, o), (o, i, t))]
    dom = gemm_by_fmt[dom_fmt]
    # per launch: a layer's dgrad and wgrad GEMMs may share one launch
    alg_bytes = sum((m * k + n * k) * ebytes + 4.0 * m * n for m, n, k in shapes) / (dom["launches"] / args.steps)
    avg_launch_s = dom["ms"] / dom["launches"] * 1e-3
    flops_per_launch = dom["flops"] / dom["launches"]
    achieved = flops_per_launch / avg_launch_s / 1e12
    from sub_byte_mixed_amd import profiling
    kernel_prefix = profiling.gemm_kernel_prefixes(dom_fmt)
    tr = profiling.load_traffic(wl.name, kernel_prefix)
    roofline = {
        "bound": "mfma",
        "kernel": (f"every {S.FORMAT_NAMES[dom_fmt]} GEMM launch: "
                   + " and ".join(k.replace("void snip::", "") + "...>" for k in kernel_prefix.split("|"))
                   + (" (fp16 MFMA after exact decode)" if dom_fmt in (S.NVFP4, S.FP8) else "")),
        "achieved": round(achieved, 2), "peak": PEAK["fp16_tflops"], "unit": "TFLOP/s",
        "frac": round(achieved / PEAK["fp16_tflops"], 4),
        "traffic": tr["traffic_bytes_per_launch"] if tr else None,
        "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "algorithmic_bytes_per_launch": round(alg_bytes),
        "avg_launch_us": round(avg_launch_s * 1e6, 2), "flops_per_launch": flops_per_launch,
        "launches_per_step": dom["launches"] // args.steps,
        "frac_of_native_peak": round(achieved / (PEAK["fp4_tflops"] if dom_fmt in (S.NVFP4, S.MXFP4)
                                                 else PEAK["fp8_tflops"]), 4),
    }
    ceil = profiling.load_mfma_ceiling()
    if ceil and dom_fmt != S.MXFP4:
        # the fp16 MFMA rate the chip sustains at the clock it holds under MFMA
        # load (about 2.0 GHz instead of the 2.4 GHz the published peak assumes)
        roofline["measured_mfma_ceiling_tflops"] = ceil["sustained_fp16_mfma_tflops"]
        roofline["frac_of_measured_ceiling"] = round(achieved / ceil["sustained_fp16_mfma_tflops"], 4)
    gemm_detail = {S.FORMAT_NAMES[f]: {"tflops": round(g["flops"] / (g["ms"] * 1e-3) / 1e12, 2),
                                       "ms_per_step": round(g["ms"] / args.steps, 4),
                                       "launches_per_step": g["launches"] // args.steps}
                   for f, g in gemm_by_fmt.items()}
    quant_gbs = quant["bytes"] / (quant["ms"] * 1e-3) / 1e9
    # The fused quantizers' ALU roofline: VALU lane-operations per element
    # (rocprofv3 SQ_INSTS_VALU, recorded with a hash of the quantizer
    # sources) times the elements each launch quantized, over the launches'
    # measured time, against the chip's full-rate VALU issue rate.
    valu = profiling.load_valu(wl.name)
    alu = None
    duals = [c for c in by_class.values() if c["dual"]]
    if valu and duals and all(c["dual"] in valu for c in duals):
        ops = sum(c["elems"] * valu[c["dual"]] for c in duals)
        ms = sum(c["ms"] for c in duals)
        achieved_ops = ops / (ms * 1e-3) / 1e12
        alu = {"bound": "alu", "kernel": "quant_dual_kernel (all formats and roundings of the step)",
               "achieved": round(achieved_ops, 2), "peak": round(profiling.VALU_LANE_OPS / 1e12, 2),
               "unit": "T VALU lane-cycles/s (cycle-weighted: quarter-rate 64-bit multiplies at their cost)",
               "frac": round(achieved_ops * 1e12 / profiling.VALU_LANE_OPS, 4),
               "lane_cycles_per_element": {" ".join(k): v for k, v in valu.items()}}

    # ------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16-mfma/fp32-acc",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T,
                   "layers": [f"{d['name']} {d['din']}->{d['dout']}" for d in layers],
                   "plan": [S.FORMAT_NAMES[d["fmt"]] for d in layers], "graph": bool(graph),
                   "quantizers": "fused: one read of X, W, dY per step" if fused else "separate passes",
                   "scaling": "delayed: tensor maxima from the previous step's statistics, no max pre-pass"
                   if args.scaling == "delayed" else "current: tensor max of each tensor (pre-pass)"},
        "gemm": gemm_detail,
        "step_ms_percentiles": pct,
        "hbm_copy_gbs": round(copy_gbs, 1),
        "quantize": {"gbs": round(quant_gbs, 1), "frac_hbm": round(quant_gbs / PEAK["hbm_gbs"], 4),
                     "frac_copy": round(quant_gbs / copy_gbs, 4),
                     "ms_per_step": round(quant["ms"] / args.steps, 4),
                     "launches_per_step": quant["launches"] // args.steps, "alu_roofline": alu},
        "other_kernels_ms_per_step": {k: round(v / args.steps, 4) for k, v in other_ms.items()},
        "memory_kernels": {k: {"ms_per_step": round(c["ms"] / args.steps, 4),
                               "launches_per_step": c["launches"] // args.steps,
                               "gbs": round(c["bytes"] / (c["ms"] * 1e-3) / 1e9, 1)}
                           for k, c in sorted(by_class.items())},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def host_info():
    """The host the oracle runs on: CPU model, cores, affinity, numpy's BLAS."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            b = libs[0]
            blas = {"library": b.get("internal_api"), "version": b.get("version"),
                    "threads": b.get("num_threads"), "architecture": b.get("architecture")}
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)), "numpy": np.__version__, "blas": blas}


def cpu_baseline(wl, rows=None, gemm_rows=None):
    """The oracle as it stands, timed on a bounded sample of the workload and
    extrapolated to one whole step.

    Quantize passes: the oracle's numpy codec (one thread). Each of the six
    passes of a layer (X, W row-wise RNE; dY row-wise SR; W, dY, X
    column-wise SR) is timed on `rows` output rows of the largest layer
    (tensor max of the whole tensor), in every format of the plan, giving
    elements/s per (format, pass kind).
    GEMMs: the oracle's fp64 reference (dequantized product and the
    elementwise bound sum|a||b|, two BLAS matmuls on all of numpy's
    threads), timed on a `gemm_rows` x `gemm_rows` block of the largest
    layer's forward GEMM at its full K, giving fp64 flop/s.
    The step estimate is every pass's elements over its measured rate plus
    every GEMM's 2*M*N*K over the measured GEMM rate."""
    import synth
    import sub_byte_mixed_amd as S
    from oracle import gemm as OG
    from oracle import quantize as OQ
    rows = rows or 2048
    gemm_rows = gemm_rows or 4096
    T = wl.tokens
    big = max(range(len(wl.layers)), key=lambda i: wl.layers[i].d_in * wl.layers[i].d_out)
    layer = wl.layers[big]
    x = synth.bf16_to_f32(synth.gen_x(wl, big))
    w = synth.bf16_to_f32(synth.gen_w(wl, big))
    dy = synth.bf16_to_f32(synth.gen_dy(wl, big))
    amax = {n: OQ.tensor_amax(t) for n, t in (("x", x), ("w", w), ("dy", dy))}
    # pass kind -> (source, layout, rounding)
    kinds = {"X row rne": ("x", 0, "rne"), "W row rne": ("w", 0, "rne"), "dY row sr": ("dy", 0, "sr"),
             "W col sr": ("w", 1, "sr"), "dY col sr": ("dy", 1, "sr"), "X col sr": ("x", 1, "sr")}
    src = {"x": x, "w": w, "dy": dy}
    rate = {}
    qsec = 0.0
    fmts = sorted(set(f for f in wl.plan if f != S.BF16))
    for fmt in fmts:
        for kind, (name, lay, rnd) in kinds.items():
            t = src[name]
            n = min(rows, t.shape[0] if lay == 0 else t.shape[1])
            ids = np.arange(n)
            t0 = time.perf_counter()
            if lay == 0:
                OQ.quantize(t[:n], fmt, rnd, 0, 8 * big, amax=amax[name], row_ids=ids)
                elems = n * t.shape[1]
            else:
                OQ.quantize_colwise(t, fmt, rnd, 0, 8 * big, amax=amax[name], col_ids=ids)
                elems = n * t.shape[0]
            dt = time.perf_counter() - t0
            qsec += dt
            rate[(fmt, kind)] = elems / dt
    # fp64 GEMM: a gemm_rows x gemm_rows block of the forward GEMM at full K
    gm = min(gemm_rows, T)
    gn = min(gemm_rows, layer.d_out)
    qa = OQ.quantize(x[:gm], wl.plan[big] if wl.plan[big] != S.BF16 else S.NVFP4, "rne", 0, 0, amax=amax["x"])
    qb = OQ.quantize(w[:gn], wl.plan[big] if wl.plan[big] != S.BF16 else S.NVFP4, "rne", 0, 1, amax=amax["w"])
    t0 = time.perf_counter()
    OG.gemm_ref(qa["xhat"], qb["xhat"])
    gsec = time.perf_counter() - t0
    gemm_rate = 2.0 * gm * gn * layer.d_in / gsec          # oracle GEMM: product + bound
    # one step of the workload at the measured rates
    t_q = 0.0
    step_flops = 0.0
    for li, l in enumerate(wl.layers):
        f = wl.plan[li]
        step_flops += 3 * 2.0 * T * l.d_in * l.d_out
        if f == S.BF16:
            continue
        n_elem = {"X": T * l.d_in, "W": l.d_out * l.d_in, "dY": T * l.d_out}
        for kind in kinds:
            t_q += n_elem[kind.split()[0]] / rate[(f, kind)]
    t_g = step_flops / gemm_rate
    info = host_info()
    return {
        "value": round(step_flops / (t_q + t_g) / 1e12, 8), "unit": "TFLOP/s",
        "cores": int((info["blas"] or {}).get("threads") or info["affinity_cores"]), "kind": "oracle",
        "sample": (f"{wl.name} {layer.name} {layer.d_in}->{layer.d_out}: each of the 6 quantize passes on "
                   f"{rows} output rows per format ({', '.join(S.FORMAT_NAMES[f] for f in fmts)}), one thread; "
                   f"the fp64 GEMM reference on a {gm}x{gn} block of its forward GEMM (K={layer.d_in}) on all "
                   f"BLAS threads; extrapolated to the whole {T}-token step "
                   f"({len(wl.layers)} layers, 6 passes and 3 GEMMs each)"),
        "seconds": round(qsec + gsec, 2),
        "step_seconds_estimate": round(t_q + t_g, 2),
        "quantize_elems_per_s_1core": {f"{S.FORMAT_NAMES[f]} {k}": round(v) for (f, k), v in rate.items()},
        "quantize_step_seconds": round(t_q, 2),
        "gemm_fp64_flops_per_s": round(gemm_rate), "gemm_note": "per 2*M*N*K of the product; the oracle "
        "also forms the bound sum|a||b|, a second fp64 matmul of the same size",
        "gemm_step_seconds": round(t_g, 2),
        "host": info,
    }


if __name__ == "__main__":
    main()
