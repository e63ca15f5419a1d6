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


def _counter_rows(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _per_dispatch(path, counter, prefix=None, contains=None):
    """{dispatch id: value} for the kernels whose name starts with `prefix`
    (or contains `contains`)."""
    out = {}
    for r in _counter_rows(path):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        if prefix is not None and not name.startswith(prefix):
            continue
        if contains is not None and contains not in name:
            continue
        out[r["Dispatch_Id"]] = out.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return out


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
    lines = [f"# HBM traffic of `{a.kernel}...` on the {a.workload} workload", "",
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
    v = sub.add_parser("vendor")
    v.add_argument("--workload", default="tinyllama1b")
    v.add_argument("--out", required=True)
    v.add_argument("--reps", type=int, default=20)
    a = ap.parse_args(argv)
    {"copy": cmd_copy, "trace": cmd_trace, "traffic": cmd_traffic, "vendor": cmd_vendor}[a.cmd_name](a)


if __name__ == "__main__":
    main()
