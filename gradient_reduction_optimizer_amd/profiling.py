"""Summaries of rocprofv3 output for this library's kernels.

    python -m gradient_reduction_optimizer_amd.profiling stats <kernel_stats.csv>
    python -m gradient_reduction_optimizer_amd.profiling traffic <fetch counter csv> <write counter csv> \\
        <copy bytes> > traffic.json
    python -m gradient_reduction_optimizer_amd.profiling counters <counter csv>

`stats` prints the per-kernel call count and average/total duration.
`counters` prints, for each of this library's kernels, the average per
dispatch of every counter in a counter_collection.csv.
`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes per
launch for each kernel, scaled by the ratio of known to counted bytes of the
plain copy kernel that ran in the same process (the calibration).
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

OURS = ("k_accumulate_window", "k_accumulate", "k_adamw", "k_norm_partials", "k_norm_final")
KERNEL_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "kernels.hip")


def short_name(name: str) -> str:
    for k in OURS:  # longest names first
        if k + "(" in name or name.endswith(k) or f"::{k}" in name:
            return k
    if "copyBuffer" in name or "copy" in name.lower():
        return "copy"
    return name[:60]


def kernel_stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["kernel | calls | avg_us | total_us | pct"]
    for r in rows:
        out.append(f"{short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}")
    return "\n".join(out)


def _per_dispatch(path: str, counter: str):
    """{kernel: [value per dispatch]} from a counter_collection.csv."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        vals[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int) -> dict:
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    # calibration: the largest copy dispatches (the probe), known bytes each way
    cf = sorted(f.get("copy", []))[-3:]
    cw = sorted(w.get("copy", []))[-3:]
    if not cf or not cw:
        raise SystemExit("no copy-kernel dispatches found for calibration")
    scale_f = copy_bytes / (sum(cf) / len(cf) * 1024)
    scale_w = copy_bytes / (sum(cw) / len(cw) * 1024)
    res = {"calibration": {"copy_bytes_each_way": copy_bytes,
                           "copy_fetch_kib": sum(cf) / len(cf), "copy_write_kib": sum(cw) / len(cw),
                           "fetch_scale": scale_f, "write_scale": scale_w},
           "kernel_source_sha256_16": hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16],
           "kernels": {}}
    for k in OURS:
        if k in f and k in w:
            fb = sum(f[k]) / len(f[k]) * 1024 * scale_f
            wb = sum(w[k]) / len(w[k]) * 1024 * scale_w
            res["kernels"][k] = {"dispatches": len(f[k]), "fetch_bytes_per_launch": fb,
                                 "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb}
    return res


def counters(path: str) -> str:
    vals = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        if k in OURS:
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in vals for c in vals[k]})
    out = ["kernel | dispatches | " + " | ".join(names)]
    for k in OURS:
        if k in vals:
            n = max(len(v) for v in vals[k].values())
            out.append(f"{k} | {n} | " + " | ".join(
                f"{sum(vals[k][c]) / len(vals[k][c]):.6g}" if vals[k][c] else "-" for c in names))
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(kernel_stats(sys.argv[2]))
    elif sys.argv[1] == "counters":
        print(counters(sys.argv[2]))
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4])), indent=1))
