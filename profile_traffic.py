#!/usr/bin/env python3
"""Collect the rocprofv3 summaries behind bench.py's roofline figures.

For one workload this runs, each as its own rocprofv3 process on bench.py:
  1. --kernel-trace --stats           per-kernel average durations
  2. --pmc FETCH_SIZE                 HBM bytes read per dispatch
  3. --pmc WRITE_SIZE                 HBM bytes written per dispatch
and the same two counters on a plain 1 GiB device-to-device copy, whose true
traffic is known, to turn counter KiB into bytes.  It writes, under
<out>/profiles/ (to be copied into the repository's profiles/ folder):
  <kernel>_<workload>_stats.md       (durations, commands)
  <kernel>_<workload>_traffic.json   (bytes per launch + source hash)
bench.py reports the stored traffic only while the HIP sources still hash to
the value recorded here.

Usage (on a GPU machine, from the repository root):
  python3 profile_traffic.py --workload elu1_bf16_b4h8n2048d64_c64 --out gpurun_out/prof
  python3 profile_traffic.py --copy-bytes 1073741824     (the calibration copy itself)
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import re
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 1 << 30


def run(cmd, log, timeout):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(timeout)] + cmd, stdout=f, stderr=subprocess.STDOUT,
                           cwd=ROOT)
    if r.returncode != 0:
        # rocprofv3 may end with a segmentation fault after the program finished; accept it when
        # the result files exist (checked by the caller)
        print(f"  (exit code {r.returncode}, see {log})", flush=True)
    return r.returncode


def short_name(kernel_name):
    m = re.search(r"(k_\w+<[^>]*>|k_\w+(?=\()|k_scan|__amd_rocclr_copyBuffer\w*)", kernel_name)
    return m.group(1) if m else kernel_name[:60]


def per_dispatch(csv_path, counter):
    """{short kernel name: [value per dispatch]} for one counter."""
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def find(path_dir, suffix):
    for dp, _, files in os.walk(path_dir):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(dp, f)
    raise FileNotFoundError(f"no *{suffix} under {path_dir}")


def copy_kernel(nbytes):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print("copied", nbytes, "bytes", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default=None)
    ap.add_argument("--out", default="gpurun_out/prof")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--copy-bytes", type=int, default=0, help="run only the calibration copy")
    args = ap.parse_args()
    if args.copy_bytes:
        copy_kernel(args.copy_bytes)
        return
    from kernelized_linear_attention_la_amd import build as hip_build
    from kernelized_linear_attention_la_amd import inputs
    import bench
    wl = inputs.WORKLOADS[args.workload]
    slot = "decode" if wl.decode_steps else ("dq" if wl.backward else "chunk")
    kernel = bench.kernel_symbol(wl, slot)
    out = os.path.join(args.out, wl.name)
    os.makedirs(out, exist_ok=True)
    rp = "rocprofv3"
    bench_cmd = ["python3", "bench.py", "--workload", wl.name, "--cpu-seconds", "0"]
    cmds = {
        "stats": [rp, "--kernel-trace", "--stats", "-f", "csv", "-d", f"{out}/stats", "-o", "run", "--"] +
                 bench_cmd + ["--steps", str(args.steps), "--warmup", "5"],
        "fetch": [rp, "--pmc", "FETCH_SIZE", "-f", "csv", "-d", f"{out}/fetch", "-o", "run", "--"] +
                 bench_cmd + ["--steps", "3", "--warmup", "1"],
        "write": [rp, "--pmc", "WRITE_SIZE", "-f", "csv", "-d", f"{out}/write", "-o", "run", "--"] +
                 bench_cmd + ["--steps", "3", "--warmup", "1"],
        "copy_fetch": [rp, "--pmc", "FETCH_SIZE", "-f", "csv", "-d", f"{out}/copy_fetch", "-o", "run", "--",
                       "python3", "profile_traffic.py", "--copy-bytes", str(COPY_BYTES)],
        "copy_write": [rp, "--pmc", "WRITE_SIZE", "-f", "csv", "-d", f"{out}/copy_write", "-o", "run", "--",
                       "python3", "profile_traffic.py", "--copy-bytes", str(COPY_BYTES)],
    }
    for name, cmd in cmds.items():
        run(cmd, f"{out}/{name}.log", 240 if name == "stats" else 120)

    # durations
    stats_csv = find(f"{out}/stats", "kernel_stats.csv")
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    # counters
    fetch = per_dispatch(find(f"{out}/fetch", "counter_collection.csv"), "FETCH_SIZE")
    write = per_dispatch(find(f"{out}/write", "counter_collection.csv"), "WRITE_SIZE")
    cf = per_dispatch(find(f"{out}/copy_fetch", "counter_collection.csv"), "FETCH_SIZE")
    cw = per_dispatch(find(f"{out}/copy_write", "counter_collection.csv"), "WRITE_SIZE")
    copy_f = max(max(v) for v in cf.values())  # the 1 GiB copy is the largest dispatch
    copy_w = max(max(v) for v in cw.values())
    scale_f = COPY_BYTES / (copy_f * 1024.0)
    scale_w = COPY_BYTES / (copy_w * 1024.0)
    kf = statistics.median(fetch[kernel])
    kw = statistics.median(write[kernel])
    bytes_per_launch = kf * 1024.0 * scale_f + kw * 1024.0 * scale_w
    if wl.decode_steps:
        alg = bench.decode_alg_bytes(wl)
    elif wl.gated:  # q, k, v read, o written, gates read
        alg = wl.B * wl.H * wl.N * ((2 * wl.dk + 2 * wl.dv) * bench.elem_bytes(wl.dtype) +
                                    4 * (wl.dk if wl.gated == "gla" else 2))
    elif wl.backward:  # Q, K, V, dO read, dQ, dK, dV written (whole backward)
        alg = wl.B * wl.H * wl.N * (3 * wl.dk + 4 * wl.dv) * bench.elem_bytes(wl.dtype)
    else:
        alg = wl.B * wl.H * wl.N * (2 * wl.dk + 2 * wl.dv) * bench.elem_bytes(wl.dtype)
    src = hip_build.source_hash(kernel)
    safe = re.sub(r"[^A-Za-z0-9]+", "_", kernel).strip("_")
    rec = {"workload": wl.name, "kernel": kernel, "source_hash": src, "bytes_per_launch": bytes_per_launch,
           "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "copy_fetch_scale": scale_f,
           "copy_write_scale": scale_w, "algorithmic_bytes_per_launch": alg,
           "traffic_over_algorithmic": bytes_per_launch / alg,
           "commands": {k: " ".join(v) for k, v in cmds.items()}}
    pdir = os.path.join(args.out, "profiles")
    os.makedirs(pdir, exist_ok=True)
    with open(os.path.join(pdir, f"{safe}_{wl.name}_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# {kernel} — {wl.name}", "",
             f"HIP source hash `{src}`. Kernel durations from `rocprofv3 --kernel-trace --stats`:", "",
             "```", cmds["stats"][0] + " " + " ".join(cmds["stats"][1:]), "```", "",
             "| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in rows:
        lines.append(f"| `{name}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.1f} |")
    lines += ["", f"HBM traffic of `{kernel}` per dispatch (median over dispatches):", "",
              f"* FETCH_SIZE {kf:.0f} KiB × {scale_f:.4f} + WRITE_SIZE {kw:.0f} KiB × {scale_w:.4f} "
              f"= {bytes_per_launch / 1e6:.2f} MB",
              f"* algorithmic bytes per launch {alg / 1e6:.2f} MB (traffic / algorithmic = "
              f"{bytes_per_launch / alg:.3f})",
              f"* scale = 1 GiB ÷ the counter on a 1 GiB torch device copy "
              f"(FETCH {copy_f:.0f} KiB, WRITE {copy_w:.0f} KiB)", "", "Commands:", "", "```"]
    for k, v in cmds.items():
        lines.append(" ".join(v))
    lines.append("```")
    with open(os.path.join(pdir, f"{safe}_{wl.name}_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
