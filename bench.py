"""Benchmark: one optimizer step of the placement-aware reduce + norm + clip +
AdamW path on one MI355X, on a synthetic 67M-parameter BF16 draft model.

A step is the whole path over one window: reduce + accumulate of every
microbatch (the headline uses one gro_accumulate_window call per window; the
same step with one gro_accumulate per microbatch is reported beside it),
gro_reduce_norm, gro_clip_adamw with the BF16 parameter copy.  Inputs
(per-microbatch BF16 gradient buckets, FP32 master/m/v) are resident in HBM
before timing starts.

Steps run back to back, so one call may find operands that the previous call
left in the 256 MB Infinity Cache.  The JSON line's "cold_cache" object
repeats both step kinds with an untimed read of an unrelated 1 GiB buffer
before every call and reports the calls' summed durations.  "attainable"
gives, for each timed kernel, the bandwidth a probe with the same access
pattern and trivial arithmetic reaches (libgro_probe.so), and the roofline
its fraction of that.

Prints ONE JSON line.  See --help for options.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
SHAPES = {
    "draft-67m": "4 layers hidden 1024, 16384x1024 embedding",
    "draft-67m-tp2-half": "4 layers hidden 1024, 8192x1024 embedding, TP2 half share",
    "dense-1b-fsdp8-shard": "one 1/8 FSDP flat shard of a 1.34B dense model",
    "hybrid-moe-4000": "4000 tensors, lognormal sizes, 70% EP-local experts",
    "dense-8b-share": "one 1e9-element FSDP shard of an 8B dense model",
}
KERNEL_SRC = os.path.join(ROOT, "gradient_reduction_optimizer_amd", "csrc", "kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")  # traffic_<workload>.json: rocprofv3 byte counters
PROBE_LIB = os.path.join(ROOT, "gradient_reduction_optimizer_amd", "libgro_probe.so")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="draft-67m")
    ap.add_argument("--cpu-sample-frac", type=float, default=1.0,
                    help="fraction of the workload's elements the oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="size of the buffer read before every call in the cold-cache timing (0: skip it)")
    ap.add_argument("--no-group", action="store_true",
                    help="skip the group-call timing (gro_accumulate_microbatches over two groups)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the streaming probes that measure what each kernel's access pattern can reach")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the benchmark, run a plain device copy of this many MiB three times "
                         "(the calibration kernel for rocprofv3 byte counters)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM traffic of `kernel` from the committed counter summary, or None if
    missing, taken on another workload or from a different kernel source."""
    try:
        with open(os.path.join(PROFILES, f"traffic_{workload}.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if not str(t.get("workload", "")).startswith(workload + " "):
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def attainable(st, n_micro: int, c_mix: int, N: int, flush, stream, log, reps: int = 20):
    """Bandwidth that each timed kernel's access pattern reaches on this
    device: libgro_probe.so moves the same arrays with the same element
    types, cache policy and chunking as the kernel but does trivial
    arithmetic.  Runs after the timed steps and overwrites the optimizer
    state arrays (which hold real optimizer-state values when it starts).
    Back to back ("GBps") and with the cache flushed before every launch
    ("GBps_cold").  None if the probe library is not built."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    V = ctypes.c_void_p
    lib.gro_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int64, V, V, V, V, V, V, ctypes.c_int, V]
    lib.gro_probe_stream.restype = ctypes.c_int
    n = (int(st.acc.numel()) // 4096) * 4096
    k = int(round(n_micro * c_mix / N))  # BF16 streams the window kernel reads per element
    # Random values like the real inputs: all-zero data streams several per
    # cent faster on this device, which would overstate the ceiling.
    gen = torch.Generator(device=st.acc.device)
    gen.manual_seed(12345)
    probe_k = k if (1 <= k <= 8 or k in (12, 16)) else 0
    g = [(torch.randn(n, generator=gen, device=st.acc.device) * 1e-2).to(torch.bfloat16)
         for _ in range(max(1, probe_k))]
    gp = (V * len(g))(*[x.data_ptr() for x in g])
    s = stream.cuda_stream
    ptrs = [st.acc.data_ptr(), st.master.data_ptr(), st.m.data_ptr(), st.v.data_ptr(), st.p_bf16.data_ptr()]

    def run(pattern, kk, nbytes, cold):
        ev = []
        for i in range(3 + reps):
            if cold:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.gro_probe_stream(pattern, n, *ptrs, gp, kk, s)
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"gro_probe_stream({pattern}) returned {rc}")
            if i >= 3:
                ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
        return nbytes * n / (ms * 1e6)

    shapes = {"k_adamw": (0, 0, 30), "k_accumulate": (2, 1, 10)}
    if probe_k:
        shapes["k_accumulate_window"] = (1, k, 2 * k + 4)
    res = {"note": "same arrays, element types, cache policy and chunking as the kernel, trivial arithmetic, "
                   "random data; k_accumulate is its later-microbatch shape (BF16 in, FP32 read and written)"}
    for name, (pattern, kk, b) in shapes.items():
        res[name] = {"GBps": run(pattern, kk, b, False)}
        if flush is not None:
            res[name]["GBps_cold"] = run(pattern, kk, b, True)
        log(f"attainable {name}: " + ", ".join(f"{key} {val:.0f}" for key, val in res[name].items()))
    del g
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, frac: float, log, windows: int = 4):
    """Time the CPU oracle (as it is) on a bounded sample of the workload:
    every non-Shard tensor plus Shard tensors in order up to `frac` of the
    elements; `windows` consecutive optimizer steps, each one full window
    (all microbatches, norm, clip, AdamW)."""
    import numpy as np
    import oracle.method as M
    from gradient_reduction_optimizer_amd import synth

    budget = frac * w.numel
    pick, total = [], 0
    for i, t in enumerate(w.tensors):
        if t.placement != "shard" or total + t.numel <= budget or not pick:
            pick.append(i)
            total += t.numel
    tensors = [w.tensors[i] for i in pick]
    owners = M.assign_owners(tensors, w.R)
    n = w.windows[0]
    master = {j: synth.master_init(w, i).numpy() for j, i in enumerate(pick)}
    m = {j: np.zeros(w.tensors[i].numel, np.float32) for j, i in enumerate(pick)}
    v = {j: np.zeros(w.tensors[i].numel, np.float32) for j, i in enumerate(pick)}
    dt = 0.0
    for step in range(1, windows + 1):
        grads = [[[synth.bf16_bits(synth.grad_bf16(w, i, 1000 * step + k, r)) for r in range(o.slots)]
                  for i, o in zip(pick, owners)] for k in range(n)]
        t0 = time.perf_counter()
        res = M.optimizer_window(owners, w.R, grads, master, m, v, w.hparams, w.max_norm, step)
        dt += time.perf_counter() - t0
        master, m, v = res.master, res.m, res.v
        del grads
    log(f"cpu oracle: {total} elements, {windows} windows of {n}, {dt:.2f} s")
    return {"value": total * windows / dt / 1e9, "unit": "Gparam updates/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(pick)} of {len(w.tensors)} tensors ({total} of {w.numel} elements), "
                      f"{windows} optimizer steps of one {n}-microbatch window each (reduce, accumulate, "
                      f"norm, clip, AdamW), numpy single-threaded, {dt:.1f} s of oracle time",
            "seconds": dt, "host": _host_cpu()}


def _host_cpu() -> dict:
    """The host the oracle ran on: CPU model and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu": model, "cores_available": cores}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only; --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    log = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))

    import torch
    from gradient_reduction_optimizer_amd import binding as B
    from gradient_reduction_optimizer_amd import synth
    from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]()
    n = w.windows[0]
    plan = Plan(w.tensors, w.R, w.bucket_elems)
    info = plan.info
    st = DeviceState(plan, "cuda:0")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    log(f"workload {w.name}: {w.numel} params, {info['n_buckets']} buckets, {info['n_chunks']} chunks, "
        f"R={w.R}, window={n}")

    # Inputs resident in HBM: one set of BF16 bucket buffers per microbatch.
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(synth.stream_seed(w.seed, 99))
    grad_tensors, grads = [], []  # keep the tensors alive: the library only gets pointers
    for k in range(n):
        bufs = st.grad_buffers()
        for b in bufs:
            b.copy_((torch.randn(b.shape, generator=gen, device="cuda:0") * w.sigma).to(torch.bfloat16))
        grad_tensors.append(bufs)
        grads.append([b.data_ptr() for b in bufs])
    st.master.copy_(torch.randn(st.master.shape, generator=gen, device="cuda:0") * w.master_sigma)
    nb = info["n_buckets"]
    acc, mp, mm, vm, pb = (st.acc.data_ptr(), st.master.data_ptr(), st.m.data_ptr(), st.v.data_ptr(),
                           st.p_bf16.data_ptr())
    torch.cuda.synchronize()

    N = info["n_owned"]
    c_mix = sum(bk["len"] * bk["slots"] for bk in plan.buckets)  # sum over elements of c
    window_ptrs = [p for k in range(n) for p in grads[k]]       # microbatch-major
    step_no = [0]

    def ev_pair():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    flush_buf = (torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda:0")
                 if args.flush_mib else None)

    def no_flush():
        pass

    def flush():
        # An untimed read of an unrelated buffer much larger than the 256 MB
        # Infinity Cache: the next call finds none of its operands cached and
        # no dirty lines of its own to write back.
        flush_buf.sum()

    def one_step(mode: str, ev, pre=no_flush):
        """One step; with `ev` (a dict of lists) a HIP event pair brackets
        every call, without it no events are recorded."""
        step_no[0] += 1

        def call(name, fn, *a):
            pre()
            e0 = ev_pair() if ev is not None else None
            fn(*a)
            if ev is not None:
                ev[name].append((e0, ev_pair()))

        if mode == "microbatch":
            for k in range(n):
                call("k_accumulate", B.gro_accumulate, plan.handle, 0, nb, grads[k], acc, k, n, s)
        elif mode == "group":
            k0 = 0
            for g in groups:
                call("k_accumulate_group", B.gro_accumulate_microbatches, plan.handle, 0, nb,
                     [p for k in range(k0, k0 + g) for p in grads[k]], k0, g, n, acc, s)
                k0 += g
        else:
            call("k_accumulate_window", B.gro_accumulate_window, plan.handle, 0, nb, window_ptrs, n, acc, s)
        call("k_norm_final", B.gro_reduce_norm, plan.handle, acc, n, s)
        call("k_adamw", B.gro_clip_adamw, plan.handle, acc, n, w.max_norm, w.hparams, step_no[0], mp, mm, vm,
             pb, s)

    def avg_ms(pairs):
        return sum(a.elapsed_time(b) for a, b in pairs) / max(len(pairs), 1)

    # Per-call events on every step would add ~4 us per event to the steps
    # they measure (~5 % of a draft-67m step), so inside the timed region
    # they are recorded on every `sample_every`-th step only.
    sample_every = max(1, args.steps // 10)

    def time_mode(mode: str) -> dict:
        """Warm up, then time exactly `steps` steps (wall clock between two
        device synchronisations); HIP events recorded on the launch stream
        around every call of every sample_every-th of these steps give the
        per-kernel durations and the per-step spread."""
        ev = {"k_accumulate": [], "k_accumulate_window": [], "k_accumulate_group": [], "k_norm_final": [],
              "k_adamw": []}
        for _ in range(args.warmup):
            one_step(mode, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            one_step(mode, ev if i % sample_every == 0 else None)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        # Per-step spread: each sampled step from its first call's start
        # event to its AdamW end event.
        first = (ev["k_accumulate"][::n] if mode == "microbatch" else
                 ev["k_accumulate_group"][::len(groups)] if mode == "group" else ev["k_accumulate_window"])
        spans = sorted(a.elapsed_time(b[1]) for (a, _), b in zip(first, ev["k_adamw"]))
        pct = lambda q: spans[min(len(spans) - 1, int(q * (len(spans) - 1) + 0.5))]
        spread = {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9)}
        norm, _, finite = B.gro_plan_get_norm(plan.handle)
        if not finite:
            raise RuntimeError("the benchmark's norm is not finite: the timed steps skipped the update")
        # algorithmic bytes per launch
        if mode == "microbatch":
            acc_launch = (n * 2 * c_mix + (4 + 8 * (n - 1)) * N) / n  # k=0: 2c+4, k>0: 2c+8 per element
            acc_name, acc_launches = "k_accumulate", n
        elif mode == "group":                                          # first group 2cg+4, later 2cg+8
            acc_launch = (n * 2 * c_mix + (4 + 8 * (len(groups) - 1)) * N) / len(groups)
            acc_name, acc_launches = "k_accumulate_group", len(groups)
        else:
            acc_launch = n * 2 * c_mix + 4 * N                         # all n microbatches + one acc write
            acc_name, acc_launches = "k_accumulate_window", 1
        kernels = {
            acc_name: {"launches_per_step": acc_launches, "avg_ms": avg_ms(ev[acc_name]),
                       "alg_bytes_per_launch": acc_launch},
            "k_adamw": {"launches_per_step": 1, "avg_ms": avg_ms(ev["k_adamw"]), "alg_bytes_per_launch": 30 * N},
            "k_norm_final": {"launches_per_step": 1, "avg_ms": avg_ms(ev["k_norm_final"])},
        }
        for k in (acc_name, "k_adamw"):
            kernels[k]["GBps"] = kernels[k]["alg_bytes_per_launch"] / (kernels[k]["avg_ms"] * 1e6)
        step_bytes = acc_launch * acc_launches + 30 * N
        dom = max((acc_name, "k_adamw"), key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches_per_step"])
        log(f"{mode}: {ms:.3f} ms/step, " + ", ".join(f"{k} {v['avg_ms'] * 1e3:.1f} us" for k, v in kernels.items()))
        return {"ms_per_step": ms, "step_ms_events": spread, "value": N / (ms * 1e-3) / 1e9,
                "kernels": kernels, "dominant": dom,
                "step_hbm": {"alg_bytes": step_bytes, "GBps": step_bytes / (ms * 1e6),
                             "frac": step_bytes / (ms * 1e6) / HBM_PEAK_GBS},
                "final_norm": norm}

    def time_cold(mode: str) -> dict:
        """The same steps with the cache flushed before every call: the sum
        of the calls' event durations, without launch gaps."""
        ev = {"k_accumulate": [], "k_accumulate_window": [], "k_norm_final": [], "k_adamw": []}
        for _ in range(2):
            one_step(mode, None, pre=flush)
        for _ in range(args.steps):
            one_step(mode, ev, pre=flush)
        torch.cuda.synchronize()
        acc_name = "k_accumulate" if mode == "microbatch" else "k_accumulate_window"
        launches = {acc_name: n if mode == "microbatch" else 1, "k_norm_final": 1, "k_adamw": 1}
        if mode == "microbatch":
            alg = {acc_name: (n * 2 * c_mix + (4 + 8 * (n - 1)) * N) / n, "k_adamw": 30 * N}
        else:
            alg = {acc_name: n * 2 * c_mix + 4 * N, "k_adamw": 30 * N}
        kernels = {}
        for k, cnt in launches.items():
            kernels[k] = {"avg_ms": avg_ms(ev[k])}
            if k in alg:
                gbs = alg[k] / (kernels[k]["avg_ms"] * 1e6)
                kernels[k].update(GBps=gbs, frac=gbs / HBM_PEAK_GBS)
        step_ms = sum(kernels[k]["avg_ms"] * cnt for k, cnt in launches.items())
        log(f"{mode} (cold cache): {step_ms:.3f} ms of calls per step, " +
            ", ".join(f"{k} {v['avg_ms'] * 1e3:.1f} us" for k, v in kernels.items()))
        return {"calls_ms_per_step": step_ms, "value": N / (step_ms * 1e-3) / 1e9, "kernels": kernels}

    groups = [n // 2, n - n // 2] if n >= 2 else [n]
    mb = time_mode("microbatch")
    grp = time_mode("group") if not args.no_group else None
    wnd = time_mode("window")
    dom = wnd["dominant"]
    achieved = wnd["kernels"][dom]["GBps"]
    out = {
        # the headline metric as stated for this benchmark: `value` is the
        # update rate; the achieved HBM GB/s and its fraction of peak are in
        # "step_hbm" (whole step) and "roofline" (dominant kernel)
        "metric": "Gparam updates/s + achieved HBM GB/s (% of peak), 67M BF16 step, 1 GPU"
                  if w.name == "draft-67m" else f"Gparam updates/s + achieved HBM GB/s (% of peak), {w.name} step, 1 GPU",
        "value": wnd["value"],
        "unit": "Gparam updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wnd["ms_per_step"],
        "step_ms_events": wnd["step_ms_events"],
        "event_sampling": f"per-call HIP events on every {sample_every}th timed step "
                          f"({len(range(0, args.steps, sample_every))} of {args.steps}); ms_per_step is the wall "
                          "clock of all timed steps",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic: BF16 grads N(0,1e-2) per microbatch, FP32 master N(0,0.02), seeded",
        "config": {"workload": f"{w.name}: {SHAPES.get(w.name, 'synthetic parameter set')}, "
                               f"{w.numel} params as this GPU's share, R={w.R} stacked rank slots, "
                               f"accumulation window {n} reduced by one gro_accumulate_window call "
                               f"(every microbatch's BF16 gradient buckets resident), global norm, "
                               f"clip {w.max_norm}, AdamW with BF16 parameter copy",
                   "params": w.numel, "R": w.R, "window": n, "bucket_elems": w.bucket_elems,
                   "n_buckets": nb, "n_chunks": info["n_chunks"], "parallelism": "single GPU share"},
        "step_hbm": wnd["step_hbm"],
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(dom, w.name)},
        "kernels": wnd["kernels"],
        "final_norm": wnd["final_norm"],
        "microbatch_call": {"note": "the same step with one gro_accumulate per microbatch (one gradient "
                                    "bucket set reused per microbatch in a real loop); bit-identical results",
                            "value": mb["value"], "ms_per_step": mb["ms_per_step"],
                            "step_ms_events": mb["step_ms_events"], "step_hbm": mb["step_hbm"],
                            "roofline_kernel": mb["dominant"],
                            "roofline_frac": mb["kernels"][mb["dominant"]]["GBps"] / HBM_PEAK_GBS,
                            "kernels": mb["kernels"]},
        "group_call": None if grp is None else {
            "note": f"the same step with gro_accumulate_microbatches over groups {groups} of the window (only a "
                    "group's buckets need to be resident); bit-identical results; k_accumulate_group is "
                    "k_accumulate_window on a group",
            "groups": groups, "value": grp["value"], "ms_per_step": grp["ms_per_step"],
            "step_hbm": grp["step_hbm"], "kernels": grp["kernels"]},
        "context": {"pages_ms_per_update_67M": [3.255, 2.624], "hardware_of_pages": "not stated"},
    }
    if flush_buf is not None:
        out["cold_cache"] = {
            "protocol": f"an untimed {args.flush_mib} MiB read of an unrelated buffer before every call; "
                        "per-call HIP event durations summed over the step (no launch gaps)",
            "window_call": time_cold("window"), "microbatch_call": time_cold("microbatch")}
    if not args.no_probe:
        try:
            att = attainable(st, n, c_mix, N, flush if flush_buf is not None else None, stream, log)
        except (OSError, RuntimeError) as e:  # the probes are context; the step timing stands without them
            log(f"attainable-bandwidth probes not run: {e}")
            att = None
        out["attainable"] = att
        for kdict in ((out["kernels"], out["microbatch_call"]["kernels"]) if att else ()):
            for name, kv in kdict.items():
                if name in att and "GBps" in kv:
                    kv["frac_of_attainable"] = kv["GBps"] / att[name]["GBps"]
        if att and dom in att:
            out["roofline"]["frac_of_attainable"] = achieved / att[dom]["GBps"]
            if "cold_cache" in out and att[dom].get("GBps_cold"):
                ck = out["cold_cache"]["window_call"]["kernels"][dom]
                ck["frac_of_attainable"] = ck["GBps"] / att[dom]["GBps_cold"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_frac, log)
    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe"] = {"bytes_read": nbytes, "bytes_written": nbytes, "launches": 3}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
