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

    python -m gradient_reduction_optimizer_amd.profiling requests <copy bytes> <counter csv>... > requests.json

`requests` counts bytes a second way, from the L2-to-fabric request counters
binned by size (TCC_EA0_RDREQ_32B/_64B/_128B for reads, TCC_EA0_WRREQ and
TCC_EA0_WRREQ_64B for writes): bytes = the sum of requests times their
size, with no calibration.  The copy kernel's counted bytes against its
known bytes check that count.  It also evaluates the gfx950 FETCH_SIZE
formula on the same run (TCC_BUBBLE counted as the 128-byte reads, every
other non-32-byte read as 64 bytes) to show where FETCH_SIZE's factor of
two comes from.  Counters may come from several passes (CSV files).
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
    if "probe_" in name:  # stream probes: kernel and template arguments, e.g. probe_window<16, 4>
        i = name.index("probe_")
        j = name.find(">", i)
        return name[i:j + 1] if j > 0 else name[i:].split("(")[0]
    if "copyBuffer" in name or "copy" in name.lower():
        return "copy"
    return name[:60]


def _ours_and_probes(names):
    """This library's kernels in OURS order, then the probe kernels sorted."""
    return [k for k in OURS if k in names] + sorted(k for k in names if k.startswith("probe_"))


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
    for k in _ours_and_probes(f.keys()):
        if k in f and k in w:
            fb = sum(f[k]) / len(f[k]) * 1024 * scale_f
            wb = sum(w[k]) / len(w[k]) * 1024 * scale_w
            res["kernels"][k] = {"dispatches": len(f[k]), "fetch_bytes_per_launch": fb,
                                 "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb}
    return res


def _per_dispatch_sums(paths):
    """{kernel: {counter: [value per dispatch]}}, values of one dispatch
    summed over the rows that report it (one row per counter instance or
    one per dispatch, as rocprofv3 writes them)."""
    acc = defaultdict(float)
    kname = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            key = (path, r["Dispatch_Id"], r["Counter_Name"])
            acc[key] += float(r["Counter_Value"])
            kname[key] = short_name(r["Kernel_Name"])
    out = defaultdict(lambda: defaultdict(list))
    for key, val in acc.items():
        out[kname[key]][key[2]].append(val)
    return out


def requests(copy_bytes: int, paths) -> dict:
    v = _per_dispatch_sums(paths)

    def avg(k, c, top=None):
        xs = v.get(k, {}).get(c, [])
        if top:
            xs = sorted(xs)[-top:]
        return sum(xs) / len(xs) if xs else None

    res = {"kernel_source_sha256_16": hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16],
           "kernels": {}}
    for k in _ours_and_probes(v.keys()) + ["copy"]:
        top = 3 if k == "copy" else None   # the calibration copies are the largest copy dispatches
        c = {name: avg(k, name, top) for name in ("TCC_EA0_RDREQ", "TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B",
                                                   "TCC_EA0_RDREQ_128B", "TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B",
                                                   "TCC_BUBBLE", "TCC_EA0_RDREQ_DRAM", "TCC_EA0_WRREQ_DRAM")}
        if c["TCC_EA0_RDREQ_128B"] is None or c["TCC_EA0_WRREQ"] is None:
            continue
        rd = 32 * c["TCC_EA0_RDREQ_32B"] + 64 * c["TCC_EA0_RDREQ_64B"] + 128 * c["TCC_EA0_RDREQ_128B"]
        wr = 32 * (c["TCC_EA0_WRREQ"] - c["TCC_EA0_WRREQ_64B"]) + 64 * c["TCC_EA0_WRREQ_64B"]
        e = {"dispatches": len(v[k]["TCC_EA0_RDREQ_128B"]), "requests_per_launch": c,
             "read_bytes_per_launch": rd, "write_bytes_per_launch": wr, "bytes_per_launch": rd + wr,
             "read_requests_binned_over_all": (c["TCC_EA0_RDREQ_32B"] + c["TCC_EA0_RDREQ_64B"] +
                                               c["TCC_EA0_RDREQ_128B"]) / c["TCC_EA0_RDREQ"]
             if c["TCC_EA0_RDREQ"] else None}
        if c["TCC_BUBBLE"] is not None:
            e["fetch_size_formula_bytes"] = (128 * c["TCC_BUBBLE"] + 32 * c["TCC_EA0_RDREQ_32B"] +
                                             64 * (c["TCC_EA0_RDREQ"] - c["TCC_BUBBLE"] - c["TCC_EA0_RDREQ_32B"]))
        if k == "copy":
            e["known_bytes_each_way"] = copy_bytes
            e["read_counted_over_known"] = rd / copy_bytes
            e["write_counted_over_known"] = wr / copy_bytes
        res["kernels"][k] = e
    return res


def counters(path: str) -> str:
    vals = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        if k in OURS or k.startswith("probe_"):
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in vals for c in vals[k]})
    out = ["kernel | dispatches | " + " | ".join(names)]
    for k in _ours_and_probes(vals.keys()):
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
    elif sys.argv[1] == "requests":
        print(json.dumps(requests(int(sys.argv[2]), sys.argv[3:]), indent=1))
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4])), indent=1))
