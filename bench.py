"""Benchmark: one step = forward + backward of every linear layer (Q, K, V, O,
Gate, Up, Down) of a Llama-like block through the quantized linear layer
(quantize X/W with round-to-nearest, GEMM; quantize dY/W/dY/X with Philox
stochastic rounding, dgrad and wgrad GEMMs; per-tensor statistics), on
synthetic bf16 inputs already resident in HBM.

Prints one JSON line: whole-step GEMM throughput (TFLOP/s over the step's
wall time, quantizers and statistics included), the dominant kernel against
its MFMA roofline, the quantizers' credited HBM bandwidth, and the CPU
oracle timed on a bounded sample on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="tinyllama1b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    ap.add_argument("--kernel-reps", type=int, default=10)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the quantized linear layer is "
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
        layers.append(d)
    torch.cuda.synchronize()

    def step():
        for li, d in enumerate(layers):
            S.linear_fwd(d["x"], d["w"], d["fmt"], seed, li, y=d["y"], stats=d["st_f"], ws=d["ws_f"])
            S.linear_bwd(d["dy"], d["x"], d["w"], d["fmt"], d["fmt"], seed, li, dx=d["dx"], dw=d["dw"],
                         stats=d["st_b"], ws=d["ws_b"], fwd_stats=d["st_f"])

    gemm_flops = sum(3 * 2 * T * d["din"] * d["dout"] for d in layers)

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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = max(e0.elapsed_time(e1), wall * 1e3) / args.steps
    value = gemm_flops / (ms_step * 1e-3) / 1e12

    # ---------------------------------------------------- per-kernel timing
    # The same GEMMs and quantize passes, launched one call at a time between
    # HIP events on the stream they run on.
    stream = torch.cuda.current_stream()
    R = args.kernel_reps

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(R):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / R * 1e-3    # seconds per call

    gemm_by_fmt = {}
    quant = {"bytes": 0.0, "sec": 0.0, "passes": 0}
    amax_sec = 0.0
    for li, d in enumerate(layers):
        fmt = d["fmt"]
        # operands exactly as the step builds them
        qx, _ = S.quantize(d["x"], S.ROWWISE, fmt, S.RNE, seed, 8 * li + 0, with_stats=False)
        qw, _ = S.quantize(d["w"], S.ROWWISE, fmt, S.RNE, seed, 8 * li + 1, with_stats=False)
        qdy, _ = S.quantize(d["dy"], S.ROWWISE, fmt, S.SR, seed, 8 * li + 2, with_stats=False)
        qwt, _ = S.quantize(d["w"], S.COLWISE, fmt, S.SR, seed, 8 * li + 3, with_stats=False)
        qdyt, _ = S.quantize(d["dy"], S.COLWISE, fmt, S.SR, seed, 8 * li + 4, with_stats=False)
        qxt, _ = S.quantize(d["x"], S.COLWISE, fmt, S.SR, seed, 8 * li + 5, with_stats=False)
        for a, b, out in ((qx, qw, d["y"]), (qdy, qwt, d["dx"]), (qdyt, qxt, d["dw"])):
            sec = timed(lambda: S.qgemm(a, b, out=out))
            g = gemm_by_fmt.setdefault(fmt, {"sec": 0.0, "flops": 0.0, "launches": 0})
            g["sec"] += sec
            g["flops"] += 2.0 * a.rows * b.rows * a.k
            g["launches"] += 1
        # quantize passes with the tensor max supplied: kernel alone
        for src, lay, rnd, qt in ((d["x"], S.ROWWISE, S.RNE, qx), (d["w"], S.ROWWISE, S.RNE, qw),
                                  (d["dy"], S.ROWWISE, S.SR, qdy), (d["w"], S.COLWISE, S.SR, qwt),
                                  (d["dy"], S.COLWISE, S.SR, qdyt), (d["x"], S.COLWISE, S.SR, qxt)):
            amax = src.abs().max().float().reshape(1)
            sec = timed(lambda: S.quantize(src, lay, fmt, rnd, seed, 1, amax=amax, out=qt,
                                           with_stats=False))
            quant["sec"] += sec
            quant["bytes"] += src.numel() * QBYTES[fmt]
            quant["passes"] += 1
    dom_fmt = max(gemm_by_fmt, key=lambda f: gemm_by_fmt[f]["sec"])
    dom = gemm_by_fmt[dom_fmt]
    avg_launch = dom["sec"] / dom["launches"]
    flops_per_launch = dom["flops"] / dom["launches"]
    achieved = flops_per_launch / avg_launch / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": f"gemm_kernel<{S.FORMAT_NAMES[dom_fmt]}> (fp16 MFMA after exact decode)"
        if dom_fmt in (S.NVFP4, S.FP8) else f"gemm_kernel<{S.FORMAT_NAMES[dom_fmt]}>",
        "achieved": round(achieved, 2), "peak": PEAK["fp16_tflops"], "unit": "TFLOP/s",
        "frac": round(achieved / PEAK["fp16_tflops"], 4), "traffic": None,
        "avg_launch_us": round(avg_launch * 1e6, 2), "flops_per_launch": flops_per_launch,
        "launches_per_step": dom["launches"],
        "frac_of_native_peak": round(achieved / (PEAK["fp4_tflops"] if dom_fmt in (S.NVFP4, S.MXFP4)
                                                 else PEAK["fp8_tflops"]), 4),
    }
    gemm_detail = {S.FORMAT_NAMES[f]: {"tflops": round(g["flops"] / g["sec"] / 1e12, 2),
                                       "ms_per_step": round(g["sec"] * 1e3, 3), "launches": g["launches"]}
                   for f, g in gemm_by_fmt.items()}
    quant_gbs = quant["bytes"] / quant["sec"] / 1e9

    # ------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16-mfma/fp32-acc",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T,
                   "layers": [f"{d['name']} {d['din']}->{d['dout']}" for d in layers],
                   "plan": [S.FORMAT_NAMES[d["fmt"]] for d in layers], "graph": bool(graph)},
        "gemm": gemm_detail,
        "quantize": {"gbs": round(quant_gbs, 1), "frac_hbm": round(quant_gbs / PEAK["hbm_gbs"], 4),
                     "ms_per_step": round(quant["sec"] * 1e3, 3), "passes": quant["passes"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(wl):
    """The oracle as it stands on a bounded sample: forward + backward of the
    first layer (Q) at the workload's format, on the first 256 tokens."""
    import synth
    from oracle import linear as OL
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    li = 0
    layer = wl.layers[li]
    Ts = min(256, wl.tokens)
    x, w, dy = synth.gen_x(wl, li, rows=Ts), synth.gen_w(wl, li), synth.gen_dy(wl, li, rows=Ts)
    x32, w32, dy32 = (synth.bf16_to_f32(t) for t in (x, w, dy))
    fmt = wl.plan[li]
    t0 = time.perf_counter()
    OL.linear_fwd(x32, w32, fmt, 0, li)
    OL.linear_bwd(dy32, x32, w32, fmt, fmt, 0, li)
    sec = time.perf_counter() - t0
    flops = 3 * 2 * Ts * layer.d_in * layer.d_out
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(sec, 2),
            "sample": f"layer {layer.name} {layer.d_in}->{layer.d_out}, T={Ts} of {wl.tokens}, "
                      f"fwd+bwd incl. all six quantize passes, format {fmt}"}


if __name__ == "__main__":
    main()
