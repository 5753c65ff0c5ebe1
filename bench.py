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
before every call and reports the calls' summed durations.  "pattern_probe"
gives, for each timed kernel, the bandwidth of a probe that moves the same
bytes with the same access pattern and trivial arithmetic (libgro_probe.so):
a reference for the kernel's arithmetic overhead, not a ceiling for other
access patterns.  With the draft-67m workload the line also carries
"dense_1b_shard": the 1B-class model's FSDP flat shard at its full window of
8 and its trailing window of 3, both call styles.

Prints ONE JSON line.  See --help for options.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the headline step")
    ap.add_argument("--only-cpu-baseline", action="store_true",
                    help="print only the CPU oracle's timing as one JSON line, without touching the GPU "
                         "(bench.py runs itself this way in a child process)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="size of the buffer read before every call in the cold-cache timing (0: skip it)")
    ap.add_argument("--no-group", action="store_true",
                    help="skip the group-call timing (gro_accumulate_microbatches over two groups)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the streaming probes that measure what each kernel's access pattern can reach")
    ap.add_argument("--no-1b", action="store_true",
                    help="with the draft-67m workload, skip the 1B-shard entry (windows 8 and 3)")
    ap.add_argument("--lib", default=None,
                    help="time this build of libgro.so instead of the in-tree one (a variant from "
                         "`python -m gradient_reduction_optimizer_amd.build --variant`)")
    ap.add_argument("--only-1b-entry", action="store_true",
                    help="print only the 1B-shard entry as one JSON line (bench.py runs itself this way in a "
                         "child process, so that the entry's buffers are the first the process allocates)")
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


def pattern_probes(st, n_micro: int, c_mix: int, N: int, flush, stream, log, reps: int = 20):
    """Bandwidth of each timed kernel's own access pattern with trivial
    arithmetic: libgro_probe.so moves the same arrays with the same element
    types, cache policy and chunking as the kernel.  It tells how much the
    kernel's arithmetic costs, not what another access pattern would reach.
    The same patterns with 8 elements per lane access (128-bit BF16, two
    128-bit FP32 accesses) are timed beside them ("wide"): the width the
    kernels do not use, for comparison.  Runs after the timed steps and
    overwrites the optimizer state arrays.  Back to back ("GBps") and with
    the cache flushed before every launch ("GBps_cold").  None if the probe
    library is not built."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    V = ctypes.c_void_p
    lib.gro_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int64, V, V, V, V, V, V, ctypes.c_int, ctypes.c_int, V]
    lib.gro_probe_stream.restype = ctypes.c_int
    n = (int(st.acc.numel()) // 4096) * 4096
    k = int(round(n_micro * c_mix / N))  # BF16 streams the window kernel reads per element
    # Random values like the real inputs: all-zero data streams several per
    # cent faster on this device, which would overstate the bandwidth.
    gen = torch.Generator(device=st.acc.device)
    gen.manual_seed(12345)
    probe_k = k if (1 <= k <= 8 or k in (12, 16)) else 0
    g = [(torch.randn(n, generator=gen, device=st.acc.device) * 1e-2).to(torch.bfloat16)
         for _ in range(max(1, probe_k))]
    gp = (V * len(g))(*[x.data_ptr() for x in g])
    s = stream.cuda_stream
    ptrs = [st.acc.data_ptr(), st.master.data_ptr(), st.m.data_ptr(), st.v.data_ptr(), st.p_bf16.data_ptr()]
    # The launch policy the library takes for a plan of this size (the rule in
    # csrc/abi.hip, acc_nontemporal, window_lds and micro_lds), so that each
    # probe runs as its kernel does: above 512 MiB of accumulator, that stream
    # moves non-temporally, and the accumulate passes run at most 2 (window
    # pass of 12 or more streams) or 3 (5 to 11 streams; per-microbatch pass)
    # workgroups per CU.
    large = int(st.acc.numel()) * 4 > (512 << 20)
    win_cap = (2 if k >= 12 else 3 if k >= 5 else 0) if large else 0
    flags = {0: int(large), 1: int(large) | (win_cap << 8), 2: int(large) | ((3 if large else 0) << 8)}

    def run(pattern, kk, nbytes, cold):
        ev = []
        for i in range(3 + reps):
            if cold:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.gro_probe_stream(pattern, n, *ptrs, gp, kk, flags.get(pattern % 3, 0) if pattern < 6 else 0, s)
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
    res = {"note": "same arrays, element types, chunking, cache policy and workgroups per CU as the kernel "
                   "on a plan of this size, trivial arithmetic, random data; k_accumulate is its later-microbatch "
                   "shape (BF16 in, FP32 read and written); 'wide': the same bytes with 8 elements per lane "
                   "access instead of the kernels' 4",
           "elements": n, "window_streams": probe_k,
           "launch": {"accumulator_nontemporal": large, "window_wg_per_cu": win_cap or None,
                      "accumulate_wg_per_cu": 3 if large else None}}
    for name, (pattern, kk, b) in shapes.items():
        res[name] = {"GBps": run(pattern, kk, b, False)}
        if flush is not None:
            res[name]["GBps_cold"] = run(pattern, kk, b, True)
        res[name]["wide"] = {"GBps": run(pattern + 3, kk, b, False)}
        if flush is not None:
            res[name]["wide"]["GBps_cold"] = run(pattern + 3, kk, b, True)
        log(f"pattern probe {name}: 4 per lane " + ", ".join(
            f"{key} {val:.0f}" for key, val in res[name].items() if key != "wide") + "; 8 per lane " +
            ", ".join(f"{key} {val:.0f}" for key, val in res[name]["wide"].items()))
    # Plain streams over the same arrays and chunking, for scale: what reading
    # only, writing only and copying reach at this size (back to back).
    res["reference_streams"] = {"read_only": run(6, 0, 4, False), "write_only": run(7, 0, 4, False),
                                "copy": run(8, 0, 8, False)}
    log("reference streams: " + ", ".join(f"{k} {v:.0f}" for k, v in res["reference_streams"].items()))
    del g
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------- CPU oracle baseline
# The oracle as it stands, timed on the host: on one core (its own
# optimizer_window, single-threaded numpy) and on every available core.  For
# the latter this harness -- not the oracle -- splits the parameters' elements
# into contiguous ranges, one per worker process, and has each worker run the
# oracle's own per-element functions (reduce, accumulate, window scale, AdamW)
# on its ranges.  The global norm is the one cross-element step: each worker
# returns the exact sum of its squares and the harness adds them exactly and
# rounds once, which is what the oracle's correctly rounded sum does, so the
# all-cores run ends in the same bits as the one-core run (checked).

def exact_sum_of_squares(g):
    """Exact sum of x*x over a float32 array, as (integer, exponent) with
    value integer * 2**exponent; None if any element is not finite.

    x = M * 2**(e - 24) with an integer M < 2**24 (frexp; FP32 has 24
    significant bits), so x*x = M*M * 2**(2e - 48).  M*M < 2**48 is split
    into two 24-bit halves, and per exponent e each half is summed by
    bincount in FP64, exactly (integers below 2**24, fewer than 2**29 of
    them, never leave the 53-bit range)."""
    import numpy as np
    x = np.asarray(g, dtype=np.float32)
    if x.size == 0:
        return 0, 0
    if not np.isfinite(x).all():
        return None
    mant, ex = np.frexp(np.abs(x).astype(np.float64))
    M = (mant * float(1 << 24)).astype(np.int64)
    sq = M * M
    e0 = int(ex.min())
    idx = (ex - e0).astype(np.int64)
    hi = np.bincount(idx, weights=(sq >> 24).astype(np.float64))
    lo = np.bincount(idx, weights=(sq & 0xFFFFFF).astype(np.float64))
    total = 0
    for j in np.nonzero((hi != 0) | (lo != 0))[0]:
        total += ((int(hi[j]) << 24) + int(lo[j])) << (2 * int(j))
    return total, 2 * (e0 - 24)


def exact_total(parts):
    """Round an exact sum of (integer, exponent) parts once to FP64."""
    from fractions import Fraction
    parts = [p for p in parts if p[0]]
    if not parts:
        return 0.0
    base = min(e for _, e in parts)
    total = sum(v << (e - base) for v, e in parts)
    return float(Fraction(total) * Fraction(2) ** base)


def _sample(w, frac: float):
    """Every non-Shard tensor plus Shard tensors in order up to `frac` of the
    workload's elements."""
    budget = frac * w.numel
    pick, total = [], 0
    for i, t in enumerate(w.tensors):
        if t.placement != "shard" or total + t.numel <= budget or not pick:
            pick.append(i)
            total += t.numel
    return pick, total


def _pieces(sizes, n_workers):
    """Split the concatenated elements of tensors with `sizes` into
    n_workers contiguous runs: per worker a list of (tensor, begin, end)
    (empty tensors are in no run)."""
    total = sum(sizes)
    bounds = [total * k // n_workers for k in range(n_workers + 1)]
    out, at = [[] for _ in range(n_workers)], 0
    for j, size in enumerate(sizes):
        for k in range(n_workers):
            a, b = max(at, bounds[k]), min(at + size, bounds[k + 1])
            if b > a:
                out[k].append((j, a - at, b - at))
        at += size
    return out


def _state_digest(pieces, master, m, v):
    import hashlib
    h = hashlib.sha256()
    for j, a, b in pieces:
        for arr in (master, m, v):
            h.update(arr[j][a:b].tobytes())
    return h.hexdigest()


def _worker(conn, pieces, owners, R, grads, master, m, v, hp, max_norm):
    """One worker's loop: phase 1 (reduce, accumulate, window scale and the
    exact norm partial of its ranges), phase 2 (AdamW on its ranges)."""
    import numpy as np
    import oracle.method as M
    st = {(j, a): [master[j][a:b].copy(), m[j][a:b].copy(), v[j][a:b].copy()] for j, a, b in pieces}
    g = {}
    while True:
        cmd = conn.recv()
        if cmd[0] == "phase1":
            n = len(grads)
            parts, bad = [], None
            for j, a, b in pieces:
                o = owners[j]
                acc = None
                for k in range(n):
                    acc = M.accumulate(acc, M.reduce_contributions(o, R, [s[a:b] for s in grads[k][j]]), k)
                g[(j, a)] = M.window_gradient(acc, n)
                if o.in_norm:
                    p = exact_sum_of_squares(g[(j, a)])
                    if p is None:
                        bad = "nan" if (bad == "nan" or np.isnan(g[(j, a)]).any()) else "inf"
                    else:
                        parts.append(p)
            conn.send((parts, bad))
        elif cmd[0] == "phase2":
            _, coef, step = cmd
            sc = M.adamw_scalars(step=step, **hp)
            for j, a, b in pieces:
                o = owners[j]
                if o.updated:
                    p, mm, vv, _ = M.adamw_update(g[(j, a)], coef, *st[(j, a)], sc, o.decayed)
                    st[(j, a)] = [p, mm, vv]
            conn.send(True)
        elif cmd[0] == "digest":
            import hashlib
            h = hashlib.sha256()
            for j, a, b in pieces:
                for arr in st[(j, a)]:
                    h.update(arr.tobytes())
            conn.send(h.hexdigest())
        else:
            conn.close()
            return


def cpu_baseline(w, frac: float, log, runs: int = 3, max_workers: int = 16):
    """Time the CPU oracle on a bounded sample of the workload (see _sample):
    one warmup window, then the median of `runs` timed windows (each a full
    optimizer step: every microbatch's reduce + accumulate, the window scale,
    the global norm, the clip coefficient and AdamW), on one core and on
    every available core (at most max_workers worker processes).  Must run
    before the process touches the GPU: the workers are forked."""
    import multiprocessing as mp
    import statistics
    import numpy as np
    import oracle.method as M
    from gradient_reduction_optimizer_amd import synth

    pick, total = _sample(w, frac)
    tensors = [w.tensors[i] for i in pick]
    owners = M.assign_owners(tensors, w.R)
    n = w.windows[0]
    t0 = time.perf_counter()
    grads = [[None if o.owner == M.EXCLUDED else
              [synth.bf16_bits(synth.grad_bf16(w, i, k, r)) for r in range(o.slots)]
              for i, o in zip(pick, owners)] for k in range(n)]
    master = {j: synth.master_init(w, i).numpy() for j, i in enumerate(pick)}
    m = {j: np.zeros(w.tensors[i].numel, np.float32) for j, i in enumerate(pick)}
    v = {j: np.zeros(w.tensors[i].numel, np.float32) for j, i in enumerate(pick)}
    log(f"cpu oracle: inputs drawn in {time.perf_counter() - t0:.1f} s")

    # one core: the oracle's optimizer_window as it is
    st1 = (dict(master), dict(m), dict(v))
    one = []
    for step in range(1, runs + 2):
        t0 = time.perf_counter()
        res = M.optimizer_window(owners, w.R, grads, *st1, w.hparams, w.max_norm, step)
        dt = time.perf_counter() - t0
        st1 = (res.master, res.m, res.v)
        if step > 1:
            one.append(dt)
    norm1 = res.norm

    # every core: worker processes over element ranges
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    nw = max(1, min(max_workers, avail))
    sizes = [w.tensors[i].numel if o.owner != M.EXCLUDED else 0 for i, o in zip(pick, owners)]
    pieces = _pieces(sizes, nw)
    ctx = mp.get_context("fork")
    conns, procs = [], []
    for k in range(nw):
        a, b = ctx.Pipe()
        p = ctx.Process(target=_worker, args=(b, pieces[k], owners, w.R, grads, master, m, v, w.hparams,
                                              w.max_norm), daemon=True)
        p.start()
        conns.append(a)
        procs.append(p)
    many = []
    try:
        for step in range(1, runs + 2):
            t0 = time.perf_counter()
            for c in conns:
                c.send(("phase1",))
            got = [c.recv() for c in conns]
            bads = [b for _, b in got if b]
            if bads:
                normN = float("nan") if "nan" in bads else float("inf")
            else:
                normN = math.sqrt(exact_total([p for parts, _ in got for p in parts]))
            coef, stepped = M.clip_coefficient(normN, w.max_norm)
            if stepped:
                for c in conns:
                    c.send(("phase2", coef, step))
                for c in conns:
                    c.recv()
            dt = time.perf_counter() - t0
            if step > 1:
                many.append(dt)
        for c in conns:
            c.send(("digest",))
        digests = [c.recv() for c in conns]
    finally:
        for c in conns:
            try:
                c.send(("stop",))
            except (BrokenPipeError, OSError):
                pass
        for p in procs:
            p.join(timeout=30)
    same = all(d == _state_digest(pieces[k], *st1) for k, d in enumerate(digests)) and normN == norm1
    if not same:
        raise RuntimeError("the all-cores oracle run did not reproduce the one-core run's bits")
    t1, tN = statistics.median(one), statistics.median(many)
    log(f"cpu oracle: {total} elements, window {n}: one core {t1:.2f} s, {nw} cores {tN:.3f} s (median of {runs})")
    host = _host_cpu()
    sample = (f"{len(pick)} of {len(w.tensors)} tensors ({total} of {w.numel} elements); one optimizer step "
              f"per run over a {n}-microbatch window (reduce, accumulate, window scale, norm, clip, AdamW); "
              f"1 warmup run, median of {runs} timed runs")
    return {"value": total / tN / 1e9, "unit": "Gparam updates/s", "cores": nw, "kind": "oracle",
            "sample": sample + f"; {nw} worker processes over element ranges, bit-identical to one core",
            "median_s": tN, "runs_s": many,
            "one_core": {"value": total / t1 / 1e9, "unit": "Gparam updates/s", "cores": 1, "kind": "oracle",
                         "sample": sample + "; the oracle's optimizer_window, single-threaded numpy",
                         "median_s": t1, "runs_s": one},
            "bit_identical_across_core_counts": same, "host": host}


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


class StepTimer:
    """One workload on the GPU: its plan and device state, every microbatch's
    BF16 gradient buckets resident in HBM (for up to `max_window`
    microbatches), and the timing of whole steps of any call style and any
    window length up to that."""

    def __init__(self, w, args, log, max_window: int, flush_buf):
        import torch
        from gradient_reduction_optimizer_amd import binding as B
        from gradient_reduction_optimizer_amd import synth
        from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan
        self.torch, self.B = torch, B
        self.w, self.args, self.log = w, args, log
        self.plan = Plan(w.tensors, w.R, w.bucket_elems)
        self.info = self.plan.info
        self.st = DeviceState(self.plan, "cuda:0")
        self.stream = torch.cuda.current_stream()
        self.s = self.stream.cuda_stream
        self.nb = self.info["n_buckets"]
        log(f"workload {w.name}: {w.numel} params, {self.nb} buckets, {self.info['n_chunks']} chunks, "
            f"R={w.R}, windows {w.windows}")
        # Inputs resident in HBM: one set of BF16 bucket buffers per microbatch.
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(synth.stream_seed(w.seed, 99))
        self.grad_tensors, self.grads = [], []  # the tensors stay alive: the library only gets pointers
        for _ in range(max_window):
            bufs = self.st.grad_buffers()
            for b in bufs:
                b.copy_((torch.randn(b.shape, generator=gen, device="cuda:0") * w.sigma).to(torch.bfloat16))
            self.grad_tensors.append(bufs)
            self.grads.append([b.data_ptr() for b in bufs])
        self.st.master.copy_(torch.randn(self.st.master.shape, generator=gen, device="cuda:0") * w.master_sigma)
        torch.cuda.synchronize()
        self.N = self.info["n_owned"]
        self.c_mix = sum(bk["len"] * bk["slots"] for bk in self.plan.buckets)  # sum over elements of c
        self.step_no = 0
        self.flush_buf = flush_buf
        # An event pair around every call adds ~4 us per event to the steps
        # it measures (~5 % of a draft-67m step), so the timed steps carry no
        # events; per-call durations come from this many further steps.
        self.event_steps = max(5, min(args.steps, 20))

    def flush(self):
        # An untimed read of an unrelated buffer much larger than the 256 MB
        # Infinity Cache: the next call finds none of its operands cached and
        # no dirty lines of its own to write back.
        self.flush_buf.sum()

    def one_step(self, mode: str, n: int, ev, groups=None, pre=None):
        """One step over a window of n microbatches; with `ev` (a dict of
        lists) a HIP event pair on the launch stream brackets every call."""
        B, s, h, acc = self.B, self.s, self.plan.handle, self.st.acc.data_ptr()
        st = self.st
        self.step_no += 1

        def mark():
            e = self.torch.cuda.Event(enable_timing=True)
            e.record(self.stream)
            return e

        def call(name, fn, *a):
            if pre is not None:
                pre()
            e0 = mark() if ev is not None else None
            fn(*a)
            if ev is not None:
                ev[name].append((e0, mark()))

        if mode == "microbatch":
            for k in range(n):
                call("k_accumulate", B.gro_accumulate, h, 0, self.nb, self.grads[k], acc, k, n, s)
        elif mode == "group":
            k0 = 0
            for g in groups:
                call("k_accumulate_group", B.gro_accumulate_microbatches, h, 0, self.nb,
                     [p for k in range(k0, k0 + g) for p in self.grads[k]], k0, g, n, acc, s)
                k0 += g
        else:
            call("k_accumulate_window", B.gro_accumulate_window, h, 0, self.nb,
                 [p for k in range(n) for p in self.grads[k]], n, acc, s)
        call("k_norm_final", B.gro_reduce_norm, h, acc, n, s)
        call("k_adamw", B.gro_clip_adamw, h, acc, n, self.w.max_norm, self.w.hparams, self.step_no,
             st.master.data_ptr(), st.m.data_ptr(), st.v.data_ptr(), st.p_bf16.data_ptr(), s)

    def alg_bytes(self, mode: str, n: int, groups=None):
        """(accumulate kernel name, launches per step, algorithmic bytes per
        launch): every gradient slot read once per microbatch; the
        accumulator written by the window's first pass, read and written by
        each later pass."""
        N, c = self.N, self.c_mix
        if mode == "microbatch":            # k = 0: 2c + 4, k > 0: 2c + 8 per element
            return "k_accumulate", n, (n * 2 * c + (4 + 8 * (n - 1)) * N) / n
        if mode == "group":                 # first group 2cg + 4, later groups 2cg + 8
            return "k_accumulate_group", len(groups), (n * 2 * c + (4 + 8 * (len(groups) - 1)) * N) / len(groups)
        return "k_accumulate_window", 1, n * 2 * c + 4 * N   # all n microbatches, one accumulator write

    def time_mode(self, mode: str, n: int, groups=None, warmup=None) -> dict:
        """Warm up (`warmup` steps, default the command line's), then time
        exactly `steps` steps, with no events, by the wall clock between two
        device synchronisations.  Then event_steps further steps with a HIP
        event pair on the launch stream around every call give the per-kernel
        durations and the per-step spread."""
        torch, args = self.torch, self.args
        ev = {"k_accumulate": [], "k_accumulate_window": [], "k_accumulate_group": [], "k_norm_final": [],
              "k_adamw": []}
        for _ in range(args.warmup if warmup is None else warmup):
            self.one_step(mode, n, None, groups)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            self.one_step(mode, n, None, groups)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        for _ in range(self.event_steps):
            self.one_step(mode, n, ev, groups)
        torch.cuda.synchronize()
        acc_name, acc_launches, acc_launch = self.alg_bytes(mode, n, groups)
        # Per-step spread: each sampled step from its first call's start
        # event to its AdamW end event.
        first = ev[acc_name][::acc_launches]
        spans = sorted(a.elapsed_time(b[1]) for (a, _), b in zip(first, ev["k_adamw"]))
        pct = lambda q: spans[min(len(spans) - 1, int(q * (len(spans) - 1) + 0.5))]
        spread = {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9)}
        norm, _, finite = self.B.gro_plan_get_norm(self.plan.handle)
        if not finite:
            raise RuntimeError("the benchmark's norm is not finite: the timed steps skipped the update")
        N = self.N
        kernels = {
            acc_name: {"launches_per_step": acc_launches, "avg_ms": _avg_ms(ev[acc_name]),
                       "alg_bytes_per_launch": acc_launch},
            "k_adamw": {"launches_per_step": 1, "avg_ms": _avg_ms(ev["k_adamw"]), "alg_bytes_per_launch": 30 * N},
            "k_norm_final": {"launches_per_step": 1, "avg_ms": _avg_ms(ev["k_norm_final"])},
        }
        for k in (acc_name, "k_adamw"):
            kernels[k]["GBps"] = kernels[k]["alg_bytes_per_launch"] / (kernels[k]["avg_ms"] * 1e6)
            kernels[k]["frac"] = kernels[k]["GBps"] / HBM_PEAK_GBS
        step_bytes = acc_launch * acc_launches + 30 * N
        dom = max((acc_name, "k_adamw"), key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches_per_step"])
        self.log(f"{self.w.name} {mode} n={n}: {ms:.3f} ms/step, " +
                 ", ".join(f"{k} {v['avg_ms'] * 1e3:.1f} us" for k, v in kernels.items()))
        return {"ms_per_step": ms, "step_ms_events": spread, "value": N / (ms * 1e-3) / 1e9,
                "kernels": kernels, "dominant": dom,
                "step_hbm": {"alg_bytes": step_bytes, "GBps": step_bytes / (ms * 1e6),
                             "frac": step_bytes / (ms * 1e6) / HBM_PEAK_GBS},
                "final_norm": norm}

    def time_graph(self, mode: str, n: int) -> dict:
        """The same step captured once in a HIP graph on a side stream and
        replayed: `warmup` untimed replays, then `steps` replays timed by the
        wall clock between two device synchronisations.  The captured step
        keeps its step count (a kernel argument); the work per replay is the
        eager step's."""
        torch, args = self.torch, self.args
        side = torch.cuda.Stream()
        side.wait_stream(self.stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        keep = (self.s, self.stream)
        try:
            with torch.cuda.graph(g, stream=side):
                self.s, self.stream = side.cuda_stream, side
                self.one_step(mode, n, None)
        finally:
            self.s, self.stream = keep
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        norm, _, finite = self.B.gro_plan_get_norm(self.plan.handle)
        if not finite:
            raise RuntimeError("the graph replays' norm is not finite")
        del g
        return {"ms_per_step": ms, "value": self.N / (ms * 1e-3) / 1e9, "final_norm": norm}

    def time_cold(self, mode: str, n: int) -> dict:
        """The same steps with the cache flushed before every call: the sum
        of the calls' event durations, without launch gaps."""
        torch = self.torch
        ev = {"k_accumulate": [], "k_accumulate_window": [], "k_norm_final": [], "k_adamw": []}
        for _ in range(2):
            self.one_step(mode, n, None, pre=self.flush)
        for _ in range(self.args.steps):
            self.one_step(mode, n, ev, pre=self.flush)
        torch.cuda.synchronize()
        acc_name, acc_launches, acc_launch = self.alg_bytes(mode, n)
        launches = {acc_name: acc_launches, "k_norm_final": 1, "k_adamw": 1}
        alg = {acc_name: acc_launch, "k_adamw": 30 * self.N}
        kernels = {}
        for k, cnt in launches.items():
            kernels[k] = {"avg_ms": _avg_ms(ev[k])}
            if k in alg:
                gbs = alg[k] / (kernels[k]["avg_ms"] * 1e6)
                kernels[k].update(GBps=gbs, frac=gbs / HBM_PEAK_GBS)
        step_ms = sum(kernels[k]["avg_ms"] * cnt for k, cnt in launches.items())
        self.log(f"{self.w.name} {mode} n={n} (cold cache): {step_ms:.3f} ms of calls per step, " +
                 ", ".join(f"{k} {v['avg_ms'] * 1e3:.1f} us" for k, v in kernels.items()))
        return {"calls_ms_per_step": step_ms, "value": self.N / (step_ms * 1e-3) / 1e9, "kernels": kernels}


def _avg_ms(pairs):
    return sum(a.elapsed_time(b) for a, b in pairs) / max(len(pairs), 1)


def _summary(r: dict, note: str) -> dict:
    """The per-step figures of one timed step kind, for a secondary entry."""
    dom = r["dominant"]
    return {"note": note, "value": r["value"], "ms_per_step": r["ms_per_step"],
            "step_ms_events": r["step_ms_events"], "step_hbm": r["step_hbm"],
            "roofline_kernel": dom, "roofline_frac": r["kernels"][dom]["frac"], "kernels": r["kernels"]}


# Steps of a freshly set-up 1B-shard plan run about 5 % slower for the
# first ~10 steps (measured: 2.06 ms, then 1.95-1.96 ms per window-call
# step), so its entry warms up at least this many steps per step kind.
MIN_WARMUP_1B = 20


def dense_1b_entry(args, log, flush_buf) -> dict:
    """The 1B-class dense model's FSDP flat shard (one GPU's eighth, R = 2
    replica slots): full window of 8 and the trailing window of 3, each with
    one gro_accumulate_window call and with one gro_accumulate per
    microbatch, plus the full window's cold-cache calls."""
    from gradient_reduction_optimizer_amd import synth
    w = synth.dense_1b_shard()
    full, trailing = w.windows
    t = StepTimer(w, args, log, full, flush_buf)
    warm = max(args.warmup, MIN_WARMUP_1B)
    out = {"workload": f"{w.name}: {SHAPES[w.name]}, {w.numel} params, R={w.R} stacked replica slots, "
                       f"buckets of {w.bucket_elems} elements, windows {w.windows}, clip {w.max_norm}, "
                       f"AdamW with BF16 parameter copy",
           "params": w.numel, "R": w.R, "windows": list(w.windows), "steps": args.steps, "warmup": warm}
    for n, label in ((full, "full_window"), (trailing, "trailing_window")):
        wnd = t.time_mode("window", n, warmup=warm)
        mb = t.time_mode("microbatch", n, warmup=warm)
        out[label] = {
            "window": n,
            "window_call": _summary(wnd, f"one gro_accumulate_window call over the {n} resident microbatches"),
            "microbatch_call": _summary(mb, f"one gro_accumulate per microbatch ({n} calls)")}
    if flush_buf is not None:
        out["full_window"]["cold_cache"] = {"window_call": t.time_cold("window", full),
                                            "microbatch_call": t.time_cold("microbatch", full)}
    if not args.no_probe:
        try:
            att = pattern_probes(t.st, full, t.c_mix, t.N, t.flush if flush_buf is not None else None,
                                 t.stream, log)
        except (OSError, RuntimeError) as e:
            log(f"pattern probes not run: {e}")
            att = None
        out["pattern_probe"] = att
        # The window and AdamW probes move exactly these kernels' bytes (the
        # accumulate probe reads one slot, this plan's kernel two).
        for kd in ((out["full_window"]["window_call"]["kernels"],) if att else ()):
            for name in ("k_accumulate_window", "k_adamw"):
                if name in kd and name in att:
                    kd[name]["frac_of_pattern_probe"] = kd[name]["GBps"] / att[name]["GBps"]
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only; --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    log = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))
    if args.lib:
        from gradient_reduction_optimizer_amd import binding
        if not os.path.exists(args.lib):
            raise SystemExit(f"--lib {args.lib}: no such library")
        binding.LIB_PATH = os.path.abspath(args.lib)

    from gradient_reduction_optimizer_amd import synth
    if args.only_1b_entry:
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        flush_buf = (torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda:0")
                     if args.flush_mib else None)
        print(json.dumps(dense_1b_entry(args, log, flush_buf)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]()
    if args.only_cpu_baseline:
        print(json.dumps(cpu_baseline(w, args.cpu_sample_frac, log)), flush=True)
        return

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    flush_buf = (torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda:0")
                 if args.flush_mib else None)
    n = w.windows[0]
    t = StepTimer(w, args, log, n, flush_buf)
    groups = [n // 2, n - n // 2] if n >= 2 else [n]
    mb = t.time_mode("microbatch", n)
    grp = t.time_mode("group", n, groups) if not args.no_group else None
    wnd = t.time_mode("window", n)
    grf = None if args.no_graph else t.time_graph("window", n)
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
        "event_sampling": f"ms_per_step is the wall clock of the {args.steps} timed steps, which carry no events; "
                          f"per-call HIP event durations and step_ms_events come from {t.event_steps} further steps "
                          "with an event pair around every call",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": f"synthetic: BF16 grads N(0,{w.sigma:g}) per microbatch, FP32 master N(0,{w.master_sigma:g}), seeded",
        "config": {"workload": f"{w.name}: {SHAPES.get(w.name, 'synthetic parameter set')}, "
                               f"{w.numel} params as this GPU's share, R={w.R} stacked rank slots, "
                               f"accumulation window {n} reduced by one gro_accumulate_window call "
                               f"(every microbatch's BF16 gradient buckets resident), global norm, "
                               f"clip {w.max_norm}, AdamW with BF16 parameter copy",
                   "params": w.numel, "R": w.R, "window": n, "bucket_elems": w.bucket_elems,
                   "n_buckets": t.nb, "n_chunks": t.info["n_chunks"], "parallelism": "single GPU share",
                   "library": os.path.relpath(args.lib, ROOT) if args.lib else "in-tree libgro.so"},
        "step_hbm": wnd["step_hbm"],
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(dom, w.name)},
        "kernels": wnd["kernels"],
        "final_norm": wnd["final_norm"],
        "microbatch_call": _summary(mb, "the same step with one gro_accumulate per microbatch (one gradient "
                                        "bucket set reused per microbatch in a real loop); bit-identical results"),
        "group_call": None if grp is None else {
            "note": f"the same step with gro_accumulate_microbatches over groups {groups} of the window (only a "
                    "group's buckets need to be resident); bit-identical results; k_accumulate_group is "
                    "k_accumulate_window on a group",
            "groups": groups, "value": grp["value"], "ms_per_step": grp["ms_per_step"],
            "step_hbm": grp["step_hbm"], "kernels": grp["kernels"]},
        "context": {"pages_ms_per_update_67M": [3.255, 2.624], "hardware_of_pages": "not stated"},
    }
    if grf is not None:
        out["graph_replay"] = {
            "note": "the headline step (window call, norm, clip + AdamW: three launches) captured once in a "
                    "HIP graph and replayed, against the same step issued eagerly",
            "ms_per_step": grf["ms_per_step"], "value": grf["value"], "eager_ms_per_step": wnd["ms_per_step"]}
    if flush_buf is not None:
        out["cold_cache"] = {
            "protocol": f"an untimed {args.flush_mib} MiB read of an unrelated buffer before every call; "
                        "per-call HIP event durations summed over the step (no launch gaps)",
            "window_call": t.time_cold("window", n), "microbatch_call": t.time_cold("microbatch", n)}
    if not args.no_probe:
        try:
            att = pattern_probes(t.st, n, t.c_mix, t.N, t.flush if flush_buf is not None else None, t.stream, log)
        except (OSError, RuntimeError) as e:  # the probes are context; the step timing stands without them
            log(f"pattern probes not run: {e}")
            att = None
        out["pattern_probe"] = att
        for kdict in ((out["kernels"], out["microbatch_call"]["kernels"]) if att else ()):
            for name, kv in kdict.items():
                if name in att and "GBps" in kv:
                    kv["frac_of_pattern_probe"] = kv["GBps"] / att[name]["GBps"]
        if att and dom in att:
            out["roofline"]["frac_of_pattern_probe"] = achieved / att[dom]["GBps"]
            if "cold_cache" in out and att[dom].get("GBps_cold"):
                ck = out["cold_cache"]["window_call"]["kernels"][dom]
                ck["frac_of_pattern_probe"] = ck["GBps"] / att[dom]["GBps_cold"]
    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe"] = {"bytes_read": nbytes, "bytes_written": nbytes, "launches": 3}
        del src, dst
    if w.name == "draft-67m" and not args.no_1b:
        del t
        flush_buf = None
        torch.cuda.empty_cache()
        out["dense_1b_shard"] = _child_or_error(dense_1b_child, args, log)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _child_or_error(cpu_baseline_child, args, log)
    print(json.dumps(out), flush=True)


def _child_or_error(fn, args, log):
    """A secondary entry measured in a child process; if that process fails,
    the line still carries the headline, with the failure stated in place of
    the entry."""
    try:
        return fn(args, log)
    except (RuntimeError, ValueError, OSError) as e:  # json.JSONDecodeError is a ValueError
        log(f"{fn.__name__}: {e}")
        return {"error": str(e)}


def cpu_baseline_child(args, log) -> dict:
    """cpu_baseline in a child process (`bench.py --only-cpu-baseline`),
    after the GPU timing.  Run inside this process before the GPU timing, the
    oracle's gigabytes of host arrays and its forked workers left the host
    slow to issue the first timed calls: the per-call events of the
    draft-67m per-microbatch steps then read 440-590 us per 90 us launch
    (the wall clock of the timed steps was unchanged)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--only-cpu-baseline", "--workload", args.workload,
           "--cpu-sample-frac", str(args.cpu_sample_frac)]
    if args.quiet:
        cmd.append("--quiet")
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"the CPU baseline's process failed with exit code {r.returncode}")
    out = json.loads(r.stdout.strip().splitlines()[-1])
    out["process"] = "timed in a child process of bench.py after the GPU timing (no GPU use)"
    return out


def dense_1b_child(args, log) -> dict:
    """The 1B-shard entry measured by this script in a child process.  In a
    process that has already allocated and freed other buffers the 1B step
    measured 1-3 % slower than in a fresh one (1.977 and 2.011 ms against
    1.956 ms per window-call step); a training job allocates its buffers
    once at start, so the fresh process is the representative one."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--only-1b-entry", "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--flush-mib", str(args.flush_mib)]
    if args.no_probe:
        cmd.append("--no-probe")
    if args.lib:
        cmd += ["--lib", args.lib]
    if args.quiet:
        cmd.append("--quiet")
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"the 1B-shard entry's process failed with exit code {r.returncode}")
    entry = json.loads(r.stdout.strip().splitlines()[-1])
    entry["process"] = "measured in a child process of bench.py (its first device allocations)"
    return entry


if __name__ == "__main__":
    main()
