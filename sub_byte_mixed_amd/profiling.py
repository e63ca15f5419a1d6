"""Measurement helpers around rocprofv3 output (host-side, no GPU needed
except for the `copy` calibration run).

  python -m sub_byte_mixed_amd.profiling copy --mib 1024 --reps 5
      runs a plain elementwise copy (torch.mul(x, 1.0, out=y), fp32) of a
      known size: the calibration kernel for FETCH_SIZE / WRITE_SIZE.
  python -m sub_byte_mixed_amd.profiling trace STATS_CSV OUT_MD --cmd "..."
      writes a short kernel-trace summary (rocprofv3 --kernel-trace --stats).
  python -m sub_byte_mixed_amd.profiling traffic --fetch F.csv --write W.csv
         --copy-fetch CF.csv --copy-write CW.csv --kernel PREFIX --copy-mib N
         --workload NAME --out OUT_MD --cmd "..."
      HBM bytes per dispatch of the kernels whose name starts with PREFIX,
      from two --pmc runs (FETCH_SIZE, then WRITE_SIZE, in KiB per
      dispatch), each scaled by the factor that makes the calibration copy
      read and write exactly its known size. The summary records a hash of
      the kernel sources, so a later change of the kernel invalidates it.
  python -m sub_byte_mixed_amd.profiling kernels --fetch F.csv --write W.csv
         --copy-fetch CF.csv --copy-write CW.csv --stats STATS_CSV
         --workload NAME --out OUT_MD --cmd "..."
      the same copy-calibrated HBM bytes for every kernel of the library,
      divided by the kernel's average duration from a kernel-trace run of
      the same command: each kernel's achieved HBM GB/s.
  python -m sub_byte_mixed_amd.profiling mfma --pmc P.csv --stats STATS_CSV
         --workload NAME --steps N --out OUT_MD --cmd "..."
      MFMA utilisation of the GEMM kernels from one --pmc run (MfmaUtil =
      MFMA-busy cycles over active cycles of all SIMDs; MFMA flops from the
      SQ_INSTS_VALU_MFMA_MOPS_* counters, 512 flops each), and the counted
      MFMA flops against the workload's 2*M*N*K over the N steps the run made.
  python -m sub_byte_mixed_amd.profiling valu --pmc P.csv --stats STATS_CSV
         --workload NAME --steps N --out OUT_MD --cmd "..."
      VALU work of the fused quantize kernels from one --pmc run: VALU
      lane-operations per element (SQ_INSTS_VALU x 64 over the elements the
      kernel quantized in the run's N steps), the element rate the chip's
      VALU issue rate allows at that count (256 CUs x 4 SIMDs x 16 lanes x
      2.4 GHz = 39.3e12 lane-operations/s), and the rate reached.
  python -m sub_byte_mixed_amd.profiling sweep --reps R
      the 7B Down projection of the precision sweep forward and backward in
      BF16, FP8, NVFP4 and MX-FP4 (1 + R repetitions each): the program the
      sweep's GEMM counter summaries are taken on.
  python -m sub_byte_mixed_amd.profiling vendor --workload NAME --out OUT_MD
      times the vendor library's fp16 and bf16 GEMM (torch.mm, hipBLASLt) on
      the workload's forward, dgrad and wgrad shapes: a reference point for
      what a tuned dense GEMM reaches at these sizes (not part of the path).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/gemm_common.h", "csrc/device.h", "csrc/kernels.h")
QUANT_SOURCES = ("csrc/quantize_dual.hip", "csrc/quant_common.h", "csrc/stats_common.h", "csrc/device.h",
                 "csrc/kernels.h")
TRAFFIC_TAG = "traffic-json:"


def source_hash(files=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read() + b"\0")
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"gemm_hbm_traffic_{workload}.md")


def load_traffic(workload: str, kernel_prefix: str):
    """Per-dispatch HBM bytes of `kernel_prefix` recorded for this workload,
    or None when absent or taken on other kernel sources."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith(TRAFFIC_TAG):
            d = json.loads(line[len(TRAFFIC_TAG):])
            if d.get("source_hash") == source_hash() and d.get("kernel") == kernel_prefix:
                return d
    return None


def load_mfma_ceiling():
    """The dense fp16 MFMA rate the chip sustains at the clock it holds under
    MFMA load (profiles/mfma_clock.md, measured by tests/helpers/mfma_clock),
    in TFLOP/s, or None."""
    path = os.path.join(ROOT, "profiles", "mfma_clock.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("mfma-clock-json:"):
            return json.loads(line[len("mfma-clock-json:"):])
    return None


def load_valu(workload: str):
    """{(format name, row rounding, column rounding): VALU lane-ops per
    element} of the fused quantize kernels recorded for this workload, or
    None when absent or taken on other quantizer sources."""
    path = os.path.join(ROOT, "profiles", f"quantize_valu_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("valu-json:"):
            d = json.loads(line[len("valu-json:"):])
            if d.get("source_hash") != source_hash(QUANT_SOURCES):
                return None
            return {tuple(k["kernel"].split(", ")): k.get("weighted_per_elem", k["ops_per_elem"]) for k in d["kernels"]}
    return None


def _counter_rows(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


def gemm_kernel_prefixes(fmt: int) -> str:
    """Kernel-name prefixes of every GEMM kernel that runs format `fmt`,
    '|'-separated: the tile kernels of gemm_kernel and, for NVFP4, the
    256x256 one-wave-per-SIMD kernel; for MX-FP4 and BF16 also the
    register-staged 128x128 kernel, and for MX-FP4 its 256x256
    one-wave-per-SIMD kernels."""
    p = [f"void snip::gemm_kernel<{fmt},"]
    if fmt == 2:
        p.append("void snip::gemm_nvfp4_w1_kernel<")
    if fmt in (0, 3):
        p.append(f"void snip::(anonymous namespace)::staged_gemm_kernel<{fmt},")
    if fmt == 3:
        p.append("snip::gemm_mxfp4_w1")
    return "|".join(p)


def _per_dispatch(path, counter, prefix=None, contains=None):
    """{dispatch id: value} for the kernels whose name starts with `prefix`
    (one of several, '|'-separated; or contains `contains`)."""
    out = {}
    prefixes = tuple(prefix.split("|")) if prefix is not None else None
    for r in _counter_rows(path):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        if prefixes is not None and not name.startswith(prefixes):
            continue
        if contains is not None and contains not in name:
            continue
        out[r["Dispatch_Id"]] = out.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return out


def _per_kernel(path, counter):
    """{kernel name: {dispatch id: value}} of one counter."""
    out = {}
    for r in _counter_rows(path):
        if r["Counter_Name"] != counter:
            continue
        d = out.setdefault(r["Kernel_Name"].strip(), {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return out


def _stats_by_name(path):
    """{kernel name: (calls, average ns)} from a --stats kernel summary."""
    return {r["Name"].strip(): (int(r["Calls"]), float(r["AverageNs"])) for r in _counter_rows(path)}


def _short(name, n=90):
    return re.sub(r"\s+", " ", name.replace("(anonymous namespace)::", ""))[:n]


def _copy_factors(a):
    cf = _per_dispatch(a.copy_fetch, "FETCH_SIZE", contains=a.copy_kernel)
    cw = _per_dispatch(a.copy_write, "WRITE_SIZE", contains=a.copy_kernel)
    if not cf or not cw:
        sys.exit("missing copy dispatches")
    known = a.copy_mib * (1 << 20)
    med = lambda v: sorted(v)[len(v) // 2]
    return known / (med(list(cf.values())) * 1024.0), known / (med(list(cw.values())) * 1024.0)


def cmd_kernels(a):
    f_r, f_w = _copy_factors(a)
    fetch = _per_kernel(a.fetch, "FETCH_SIZE")
    write = _per_kernel(a.write, "WRITE_SIZE")
    stats = _stats_by_name(a.stats)
    rows = []
    for name, fd in fetch.items():
        if not name.startswith("void snip::") and not name.startswith("snip::"):
            continue
        wd = write.get(name)
        if not wd or name not in stats:
            continue
        rd = sum(fd.values()) / len(fd) * 1024 * f_r
        wr = sum(wd.values()) / len(wd) * 1024 * f_w
        calls, avg_ns = stats[name]
        rows.append((name, len(fd), rd, wr, avg_ns, (rd + wr) / avg_ns))
    rows.sort(key=lambda r: -r[1] * r[4])
    # bf16 input bytes per dispatch of the fused quantizers (one read of X, W, dY per step)
    sys.path.insert(0, ROOT)
    import synth
    elems = dual_elements_per_step(synth.WORKLOADS[a.workload])
    launches = {}
    for l, f in zip(synth.WORKLOADS[a.workload].layers, synth.WORKLOADS[a.workload].plan):
        for key in ((f, False, True), (f, True, True)):
            launches[key] = launches.get(key, 0) + 1

    def input_mb(name):
        m = re.search(r"quant_dual_kernel<(\d+), (true|false), (true|false)>", name)
        if not m:
            return "-"
        key = (int(m.group(1)), m.group(2) == "true", m.group(3) == "true")
        return f"{2.0 * elems[key] / launches[key] / 1e6:.2f}"
    lines = [f"# HBM bytes and achieved HBM GB/s of every kernel on the {a.workload} workload", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, two --pmc runs of the benchmark), each scaled",
             f"by the factor that makes a plain fp32 copy of {a.copy_mib} MiB read and write exactly its size",
             f"(read {f_r:.4f}, write {f_w:.4f}); GB/s = bytes per dispatch over the kernel's average",
             "duration in a kernel-trace run of the same benchmark (same launches per step). HBM peak 8000",
             "GB/s. Commands (from the repository root):", "", "```", a.cmd, "```", "",
             "The fused quantizers' bf16 input per dispatch (X and W of a layer, or its dY) is listed beside",
             "the bytes they fetch: each tensor is read once.", "",
             "| Kernel | Dispatches | Read MB / dispatch | bf16 input MB / dispatch | Written MB / dispatch | "
             "Average us (trace) | HBM GB/s | of peak |",
             "|---|---|---|---|---|---|---|---|"]
    for name, n, rd, wr, ns, gbs in rows:
        lines.append(f"| `{_short(name)}` | {n} | {rd / 1e6:.2f} | {input_mb(name)} | {wr / 1e6:.2f} | {ns / 1e3:.2f} | "
                     f"{gbs:.0f} | {gbs / 8000 * 100:.1f} % |")
    lines.append("")
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def cmd_mfma(a):
    sys.path.insert(0, ROOT)
    import synth
    wl = synth.WORKLOADS[a.workload]
    flops_step = sum(3 * 2 * wl.tokens * l.d_in * l.d_out for l in wl.layers)
    util = _per_kernel(a.pmc, "MfmaUtil")
    mops = {k: _per_kernel(a.pmc, f"SQ_INSTS_VALU_MFMA_MOPS_{k}") for k in ("F16", "BF16", "F6F4", "F8")}
    grbm = _per_kernel(a.pmc, "GRBM_GUI_ACTIVE")
    stats = _stats_by_name(a.stats) if a.stats else {}
    res = {}
    for r in _counter_rows(a.pmc):
        res.setdefault(r["Kernel_Name"].strip(), r["LDS_Block_Size"])
    lines = [f"# MFMA utilisation of the GEMM kernels on the {a.workload} workload", "",
             "One rocprofv3 --pmc run of the benchmark. MfmaUtil (rocprofv3's derived counter) = MFMA-busy",
             "cycles summed over the SIMDs / (active GPU cycles x SIMDs), per dispatch, averaged over the",
             "kernel's dispatches. MFMA TFLOP per dispatch = SQ_INSTS_VALU_MFMA_MOPS_* x 512. Commands (from",
             "the repository root):", "", "```", a.cmd, "```", "",
             "| Kernel | Dispatches | MfmaUtil % | MFMA GFLOP / dispatch (counted) | MFMA type | Average us (trace) | "
             "LDS bytes |", "|---|---|---|---|---|---|---|"]
    total = 0.0
    for name in sorted(util, key=lambda n: -sum(util[n].values())):
        if not _is_gemm(name):
            continue
        ud = util[name]
        fl = {k: sum(m.get(name, {}).values()) * 512 for k, m in mops.items()}
        kind = max(fl, key=fl.get)
        n = len(ud)
        total += sum(fl.values())
        avg = f"{stats[name][1] / 1e3:.2f}" if name in stats else "-"
        lines.append(f"| `{_short(name)}` | {n} | {sum(ud.values()) / n:.1f} | {fl[kind] / n / 1e9:.2f} | {kind} | {avg} | "
                     f"{res.get(name, '-')} |")
    lines += ["", f"Counted MFMA flops over all GEMM dispatches: {total:.6e}; the workload's 2*M*N*K over the "
              f"run's {a.steps} steps: {flops_step * a.steps:.6e} (ratio {total / (flops_step * a.steps):.6f}).",
              ""]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def _is_gemm(name: str) -> bool:
    """A GEMM kernel of the library, in a named or an anonymous namespace
    (gemm_kernel, staged_gemm_kernel, gemm_nvfp4_w1_kernel, ...)."""
    return "snip::" in name and re.search(r"\bgemm_|staged_gemm_", name) is not None


def cmd_stalls(a):
    """Where the GEMM kernels' wave time goes: SQ wave-cycle counters of
    several --pmc runs, each as a share of SQ_WAVE_CYCLES taken in the same
    run (all in quad-cycles, summed over the kernel's dispatches)."""
    rows = []                   # (counter, {kernel: share})
    for path in a.pmc:
        names = sorted({r["Counter_Name"] for r in _counter_rows(path)})
        wave = _per_kernel(path, "SQ_WAVE_CYCLES")
        for c in names:
            if c == "SQ_WAVE_CYCLES":
                continue
            vals = _per_kernel(path, c)
            rows.append((c, {k: sum(v.values()) / max(sum(wave.get(k, {}).values()), 1.0) for k, v in vals.items()}))
    kernels = sorted({k for _, d in rows for k in d if _is_gemm(k)})
    head = "| Counter / SQ_WAVE_CYCLES | " + " | ".join(f"`{_short(k, 48)}`" for k in kernels) + " |"
    lines = [f"# Wave-cycle breakdown of the GEMM kernels on the {a.workload} workload", "",
             "SQ counters in quad-cycles, summed over each kernel's dispatches in a --pmc run of the benchmark,",
             "divided by SQ_WAVE_CYCLES of the same run: WAIT_ANY = waves waiting on a dependency (s_waitcnt,",
             "barrier), WAIT_INST_ANY = waves with an instruction ready but not issued, ACTIVE_INST_* = waves",
             "issuing that instruction type. Shares of a wave's time; with several waves per SIMD they overlap.",
             "Commands (from the repository root):", "", "```", a.cmd, "```", "", head,
             "|---|" + "---|" * len(kernels)]
    for c, d in rows:
        lines.append(f"| {c} | " + " | ".join(f"{100 * d.get(k, 0.0):.1f} %" for k in kernels) + " |")
    lines.append("")
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9      # lane-operations per second, full-rate VALU


def dual_elements_per_step(wl):
    """Elements each fused quantize kernel family (format, row SR, column
    SR) reads per step of the saved-operand layer calls: X and W once in the
    forward (nearest row-wise, stochastic column-wise), dY once in the
    backward (stochastic both ways)."""
    out = {}
    for l, f in zip(wl.layers, wl.plan):
        fwd = (f, False, True)
        bwd = (f, True, True)
        out[fwd] = out.get(fwd, 0) + wl.tokens * l.d_in + l.d_out * l.d_in
        out[bwd] = out.get(bwd, 0) + wl.tokens * l.d_out
    return out


def cmd_valu(a):
    """VALU work of the fused quantizers, counted two ways: instructions
    (SQ_INSTS_VALU, each a full-rate slot) and issue cycles
    (SQ_ACTIVE_INST_VALU, in quad-cycles per wave: quarter-rate 64-bit
    multiplies such as Philox's v_mad_u64_u32 count their real cost). The
    cycle-weighted count is the one the VALU roofline uses."""
    sys.path.insert(0, ROOT)
    import synth
    wl = synth.WORKLOADS[a.workload]
    elems = dual_elements_per_step(wl)
    insts = _per_kernel(a.pmc, "SQ_INSTS_VALU")
    int64 = _per_kernel(a.pmc, "SQ_INSTS_VALU_INT64")
    active = _per_kernel(a.pmc, "SQ_ACTIVE_INST_VALU")
    busy = _per_kernel(a.pmc, "VALUBusy")
    stats = _stats_by_name(a.stats)
    names = {0: "bf16", 1: "fp8_e4m3", 2: "nvfp4", 3: "mxfp4"}
    lines = [f"# VALU work of the fused quantize kernels on the {a.workload} workload", "",
             "One rocprofv3 --pmc run of the benchmark. Per element of the kernel family (X and W in the",
             f"forward, dY in the backward, one read each; the run's {a.steps} steps):",
             "- lane-ops = SQ_INSTS_VALU x 64 (every VALU instruction one slot);",
             "- of which int64 = SQ_INSTS_VALU_INT64 x 64 (Philox's 32x32->64-bit multiplies, quarter rate,",
             "  and 64-bit index arithmetic);",
             "- lane-cycles = SQ_ACTIVE_INST_VALU x 4 cycles x 16 lanes (the cycles the SIMDs spend issuing",
             "  VALU work, multi-cycle instructions at their real cost): the cycle-weighted count.",
             "VALU-bound rate = 39.3e12 lane-slots/s (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz) over the",
             "cycle-weighted count; reached = elements per dispatch over the average duration of a",
             "kernel-trace run of the same benchmark. VALUBusy is rocprofv3's derived counter (the SIMDs'",
             "VALU issue cycles over elapsed cycles). Commands (from the repository root):", "", "```", a.cmd,
             "```", "",
             "| Kernel (format, row rounding, column rounding) | Dispatches | VALU lane-ops / elem | int64 / elem | "
             "lane-cycles / elem | VALUBusy % | VALU-bound Gelem/s | reached Gelem/s | of VALU bound |",
             "|---|---|---|---|---|---|---|---|---|"]
    out = []
    for name, d in insts.items():
        m = re.search(r"quant_dual_kernel<(\d+), (true|false), (true|false)>", name)
        if not m:
            continue
        key = (int(m.group(1)), m.group(2) == "true", m.group(3) == "true")
        n = len(d)
        e_total = elems[key] * a.steps
        ops = sum(d.values()) * 64 / e_total
        i64 = sum(int64.get(name, {}).values()) * 64 / e_total
        cyc = sum(active.get(name, {}).values()) * 4 * 16 / e_total
        weighted = cyc if cyc > 0 else ops
        bound = VALU_LANE_OPS / weighted / 1e9
        calls, avg_ns = stats[name]
        reached = e_total / n / avg_ns
        vb = sum(busy.get(name, {}).values()) / max(1, len(busy.get(name, {})))
        label = f"{names[key[0]]}, {'SR' if key[1] else 'RNE'}, {'SR' if key[2] else 'RNE'}"
        out.append({"kernel": label, "ops_per_elem": round(ops, 2), "int64_per_elem": round(i64, 2),
                    "cycles_per_elem": round(cyc, 2), "weighted_per_elem": round(weighted, 2),
                    "valu_busy": round(vb, 1), "bound_gelem_s": round(bound, 1),
                    "reached_gelem_s": round(reached, 1)})
        lines.append(f"| `quant_dual_kernel` {label} | {n} | {ops:.1f} | {i64:.1f} | {cyc:.1f} | {vb:.1f} | "
                     f"{bound:.0f} | {reached:.0f} | {reached / bound * 100:.1f} % |")
    lines += ["", "valu-json:" + json.dumps({"workload": a.workload, "source_hash": source_hash(QUANT_SOURCES),
                                              "kernels": out}), ""]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def copy_bandwidth(torch, dev, mib: int = 1024, reps: int = 10) -> float:
    """Measured device-to-device copy rate (GB/s, bytes read + written) of a
    plain torch copy of `mib` MiB, the median of `reps`: the practical HBM
    ceiling the quantizers are also compared with."""
    a = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    return 2.0 * (mib << 20) / (sorted(ts)[reps // 2] * 1e-3) / 1e9


def cmd_copy(a):
    import torch
    n = a.mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "reps": a.reps}), flush=True)


def cmd_trace(a):
    rows = _counter_rows(a.stats_csv)
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# Kernel trace: {a.title}", "", "Command (from the repository root):", "",
             "```", a.cmd, "```", "",
             "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows[: a.top]:
        name = re.sub(r"\s+", " ", r["Name"])[:110]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / total * 100:.2f} % |")
    lines.append("")
    with open(a.out_md, "w") as fh:
        fh.write("\n".join(lines))
    print(a.out_md)


def cmd_traffic(a):
    fetch = _per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write = _per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cf = _per_dispatch(a.copy_fetch, "FETCH_SIZE", contains=a.copy_kernel)
    cw = _per_dispatch(a.copy_write, "WRITE_SIZE", contains=a.copy_kernel)
    if not fetch or not write or not cf or not cw:
        sys.exit(f"missing dispatches: fetch {len(fetch)} write {len(write)} copy {len(cf)}/{len(cw)}")
    known = a.copy_mib * (1 << 20)
    # calibration: median copy dispatch (KiB) against the known bytes
    med = lambda v: sorted(v)[len(v) // 2]
    f_r = known / (med(list(cf.values())) * 1024.0)
    f_w = known / (med(list(cw.values())) * 1024.0)
    mf = sum(fetch.values()) / len(fetch)
    mw = sum(write.values()) / len(write)
    d = {"kernel": a.kernel, "workload": a.workload, "dispatches": [len(fetch), len(write)],
         "fetch_kib_per_dispatch": round(mf, 1), "write_kib_per_dispatch": round(mw, 1),
         "copy_kib": [round(med(list(cf.values())), 1), round(med(list(cw.values())), 1)],
         "copy_bytes": known, "factor_read": round(f_r, 4), "factor_write": round(f_w, 4),
         "read_bytes_per_launch": round(mf * 1024 * f_r), "write_bytes_per_launch": round(mw * 1024 * f_w),
         "traffic_bytes_per_launch": round(mf * 1024 * f_r + mw * 1024 * f_w),
         "source_hash": source_hash()}
    names = " and ".join(f"`{k}...`" for k in a.kernel.split("|"))
    lines = [f"# HBM traffic of {names} on the {a.workload} workload", "",
             "Two rocprofv3 `--pmc` runs of the benchmark (FETCH_SIZE, then WRITE_SIZE; KiB per",
             "dispatch, averaged over the kernel's dispatches), each scaled by the factor that makes",
             f"a plain fp32 elementwise copy of {a.copy_mib} MiB (`torch.mul(x, 1.0, out=y)`) read and",
             "write exactly its size. Commands (from the repository root):", "", "```", a.cmd, "```", "",
             f"- dispatches: {d['dispatches'][0]} (FETCH_SIZE run), {d['dispatches'][1]} (WRITE_SIZE run)",
             f"- FETCH_SIZE {mf:.1f} KiB/dispatch, WRITE_SIZE {mw:.1f} KiB/dispatch",
             f"- copy: FETCH_SIZE {d['copy_kib'][0]} KiB, WRITE_SIZE {d['copy_kib'][1]} KiB for {known} bytes "
             f"each way: factors {f_r:.4f} (read), {f_w:.4f} (write)",
             f"- HBM traffic per launch: {d['read_bytes_per_launch']:,} B read + "
             f"{d['write_bytes_per_launch']:,} B written = {d['traffic_bytes_per_launch']:,} B",
             "", TRAFFIC_TAG + json.dumps(d), ""]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps(d))


def cmd_vendor(a):
    import torch
    sys.path.insert(0, ROOT)
    import synth
    wl = synth.WORKLOADS[a.workload]
    T = wl.tokens
    shapes = []
    for l in wl.layers:
        shapes += [(T, l.d_out, l.d_in), (T, l.d_in, l.d_out), (l.d_out, l.d_in, T)]
    lines = [f"# Vendor dense GEMM on the {a.workload} GEMM shapes (reference point)", "",
             "torch.mm(a, b.t()) with a [M][K] and b [N][K] (the library's operand layout), the",
             "ROCm PyTorch build's hipBLASLt path; 3 warm-up calls, then the mean of "
             f"{a.reps} back-to-back calls", "timed with HIP events. Command (from the repository root):", "",
             "```", f"python -m sub_byte_mixed_amd.profiling vendor --workload {a.workload} --out {a.out}", "```",
             "", "| dtype | M | N | K | us | TFLOP/s |", "|---|---|---|---|---|---|"]
    summary = {}
    for dt in (torch.float16, torch.bfloat16):
        fl, us_tot = 0.0, 0.0
        for (M, N, K) in shapes:
            x = torch.randn(M, K, device="cuda").to(dt)
            y = torch.randn(N, K, device="cuda").to(dt)
            for _ in range(3):
                torch.mm(x, y.t())
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(a.reps):
                torch.mm(x, y.t())
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / a.reps * 1e3
            fl += 2.0 * M * N * K
            us_tot += us
            lines.append(f"| {str(dt)[6:]} | {M} | {N} | {K} | {us:.1f} | {2.0 * M * N * K / us / 1e6:.0f} |")
        summary[str(dt)[6:]] = round(fl / us_tot / 1e6, 1)
        print(f"{dt}: {summary[str(dt)[6:]]} TFLOP/s over the step's GEMMs", flush=True)
    lines += ["", "Aggregate over the step's GEMM shapes (total flops / total time): " +
              ", ".join(f"{k} {v} TFLOP/s" for k, v in summary.items()), ""]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines))
    print(a.out)


def cmd_sweep(a):
    """The 7B Down projection of the precision sweep (T = 16384, 11008 ->
    4096) forward and backward in every format of the sweep (BF16, FP8,
    NVFP4, MX-FP4), one warm-up and `reps` timed repetitions each: the
    program the sweep's GEMM counter summaries are taken on. Prints each
    format's GEMM TFLOP/s (launch timing) against its MFMA peak."""
    sys.path.insert(0, ROOT)
    import torch
    import synth
    import sub_byte_mixed_amd as S
    wl = synth.WORKLOADS["down7b_sweep"]
    x, w, dy = (t.cuda() for t in synth.gen_layer(wl, 0))
    peak = {S.BF16: 2516.6e12, S.FP8: 2516.6e12, S.NVFP4: 2516.6e12, S.MXFP4: 10066.3e12}
    for fmt in (S.BF16, S.FP8, S.NVFP4, S.MXFP4):
        for rep in range(a.reps + 1):
            if rep == 1:
                torch.cuda.synchronize()
                S.timing_start(4096)
            S.linear_fwd(x, w, fmt, 0, 0)
            S.linear_bwd(dy, x, w, fmt, fmt, 0, 0)
        recs, _ = S.timing_read()
        g = [r for r in recs if r["kind"] == "gemm"]
        fl, ms = sum(r["work"] for r in g), sum(r["ms"] for r in g)
        print(f"{S.FORMAT_NAMES[fmt]}: {len(g)} GEMM launches, {fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s, "
              f"{fl / (ms * 1e-3) / peak[fmt] * 100:.1f} % of its MFMA peak", flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out_md")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--top", type=int, default=25)
    f = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "workload", "out", "cmd"):
        f.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    f.add_argument("--copy-kernel", default="MulFunctor", help="substring of the copy kernel's name")
    f.add_argument("--copy-mib", type=int, default=1024)
    k = sub.add_parser("kernels")
    for key in ("fetch", "write", "copy_fetch", "copy_write", "stats", "workload", "out", "cmd"):
        k.add_argument("--" + key.replace("_", "-"), dest=key, required=True)
    k.add_argument("--copy-kernel", default="MulFunctor")
    k.add_argument("--copy-mib", type=int, default=1024)
    m = sub.add_parser("mfma")
    for key in ("pmc", "workload", "out", "cmd"):
        m.add_argument("--" + key, dest=key, required=True)
    m.add_argument("--stats", default=None)
    m.add_argument("--steps", type=int, required=True, help="steps the profiled run made (warmup + 2 * steps)")
    q = sub.add_parser("valu")
    for key in ("pmc", "stats", "workload", "out", "cmd"):
        q.add_argument("--" + key, dest=key, required=True)
    q.add_argument("--steps", type=int, required=True, help="steps the profiled run made (warmup + 2 * steps)")
    w = sub.add_parser("stalls")
    w.add_argument("--pmc", nargs="+", required=True)
    for key in ("workload", "out", "cmd"):
        w.add_argument("--" + key, dest=key, required=True)
    sw = sub.add_parser("sweep")
    sw.add_argument("--reps", type=int, default=3)
    v = sub.add_parser("vendor")
    v.add_argument("--workload", default="tinyllama1b")
    v.add_argument("--out", required=True)
    v.add_argument("--reps", type=int, default=20)
    a = ap.parse_args(argv)
    {"copy": cmd_copy, "trace": cmd_trace, "traffic": cmd_traffic, "kernels": cmd_kernels, "mfma": cmd_mfma,
     "valu": cmd_valu, "stalls": cmd_stalls, "sweep": cmd_sweep,
     "vendor": cmd_vendor}[a.cmd_name](a)


if __name__ == "__main__":
    main()
