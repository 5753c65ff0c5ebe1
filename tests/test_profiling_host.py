"""Host tests of the rocprofv3 summary helpers and bench.py's argument
handling (no GPU needed).  The CSV rows below are hand-made fixtures in
rocprofv3's column layout, not measurements."""
import csv
import json
import os
import subprocess
import sys

import pytest

from gradient_reduction_optimizer_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": kernel,
                        "Counter_Name": counter, "Counter_Value": value})


def test_short_names_tell_the_two_accumulate_kernels_apart():
    assert P.short_name("gro::(anonymous namespace)::k_accumulate_window(gro::WindowLaunch)") == \
        "k_accumulate_window"
    assert P.short_name("gro::(anonymous namespace)::k_accumulate(gro::AccumulateLaunch)") == "k_accumulate"
    assert P.short_name("gro::(anonymous namespace)::k_adamw(gro::AdamWLaunch)") == "k_adamw"
    assert P.short_name("void at::native::copy_kernel_impl(...)") == "copy"


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path):
    copy = "void at::native::elementwise_copy_kernel(...)"
    adam = "gro::(anonymous namespace)::k_adamw(gro::AdamWLaunch)"
    # a 1 MiB copy whose fetch counter reads half the bytes and whose write
    # counter reads them all; AdamW dispatches read 100 / 300 KiB, write 50
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    _counter_csv(fetch, [(copy, "FETCH_SIZE", 512.0)] * 3 +
                 [(adam, "FETCH_SIZE", 100.0), (adam, "FETCH_SIZE", 300.0)])
    _counter_csv(write, [(copy, "WRITE_SIZE", 1024.0)] * 3 +
                 [(adam, "WRITE_SIZE", 50.0), (adam, "WRITE_SIZE", 50.0)])
    t = P.traffic(str(fetch), str(write), 1 << 20)
    assert t["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert t["calibration"]["write_scale"] == pytest.approx(1.0)
    k = t["kernels"]["k_adamw"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2.0)
    assert k["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    assert k["bytes_per_launch"] == pytest.approx(k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"])


def test_traffic_needs_a_calibration_copy(tmp_path):
    adam = "gro::(anonymous namespace)::k_adamw(gro::AdamWLaunch)"
    f = tmp_path / "f.csv"
    _counter_csv(f, [(adam, "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        P.traffic(str(f), str(f), 1 << 20)


def test_counter_averages_per_kernel(tmp_path):
    win = "gro::(anonymous namespace)::k_accumulate_window(gro::WindowLaunch)"
    f = tmp_path / "c.csv"
    _counter_csv(f, [(win, "SQ_WAVES", 4.0), (win, "SQ_WAVES", 8.0), (win, "SQ_INSTS_VALU", 10.0),
                     ("void at::native::reduce_kernel(...)", "SQ_WAVES", 99.0)])
    lines = P.counters(str(f)).splitlines()
    assert lines[0] == "kernel | dispatches | SQ_INSTS_VALU | SQ_WAVES"
    assert lines[1] == "k_accumulate_window | 2 | 10 | 6"
    assert len(lines) == 2


def test_probe_library_exports_its_entry_point():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gradient_reduction_optimizer_amd", "libgro_probe.so"))
    assert hasattr(lib, "gro_probe_stream")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_times_the_cpu_oracle_without_the_gpu():
    """The CPU baseline's own mode (the child process bench.py starts after
    its GPU timing) prints one JSON line and touches no GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--only-cpu-baseline", "--workload",
                        "tiny-literal", "--quiet"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["kind"] == "oracle" and out["bit_identical_across_core_counts"] is True
    assert out["one_core"]["cores"] == 1 and out["value"] > 0


def test_a_failed_child_entry_is_reported_in_the_line():
    sys.path.insert(0, ROOT)
    import bench

    def fails(args, log):
        raise RuntimeError("the child's process failed with exit code 134")

    got = bench._child_or_error(fails, None, lambda *a: None)
    assert got == {"error": "the child's process failed with exit code 134"}
    assert bench._child_or_error(lambda args, log: {"value": 1.0}, None, lambda *a: None) == {"value": 1.0}


def test_exact_sum_of_squares_matches_a_correctly_rounded_sum():
    """bench.py's all-cores oracle timing adds the workers' norm partials
    exactly; rounded once, that must equal math.fsum of the squares (the
    oracle's own correctly rounded sum) bit for bit, here on values that
    span the FP32 range: subnormals, huge values, zeros, mixed signs."""
    import math
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    rng = np.random.default_rng(5)
    cases = [rng.standard_normal(10_000).astype(np.float32) * 1e-2,
             (rng.standard_normal(5_000) * np.exp2(rng.integers(-140, 60, 5_000))).astype(np.float32),
             np.array([0.0, -0.0, 1.0, np.float32(2.0 ** -149), -3.5e18], np.float32),
             np.zeros(7, np.float32), np.zeros(0, np.float32)]
    for x in cases:
        want = math.fsum(float(t) * float(t) for t in x.astype(np.float64))
        got = bench.exact_total([bench.exact_sum_of_squares(x)])
        assert got == want, (got, want)
        # the same sum split into uneven parts
        cuts = sorted(rng.integers(0, x.size + 1, 3)) if x.size else []
        parts = [bench.exact_sum_of_squares(p) for p in np.split(x, cuts)]
        assert bench.exact_total(parts) == want
    assert bench.exact_sum_of_squares(np.array([1.0, np.inf], np.float32)) is None


def test_all_cores_oracle_timing_reproduces_one_core_bits():
    """The all-cores timing harness ends in the same bits as the oracle's own
    optimizer_window on one core (it raises otherwise), on the tiny set."""
    sys.path.insert(0, ROOT)
    import bench
    from gradient_reduction_optimizer_amd import synth
    r = bench.cpu_baseline(synth.tiny(literal=True), 1.0, lambda *a: None, runs=3, max_workers=3)
    assert r["bit_identical_across_core_counts"] is True
    assert r["cores"] == min(3, len(os.sched_getaffinity(0)))
    assert r["one_core"]["cores"] == 1 and len(r["runs_s"]) == 3 and len(r["one_core"]["runs_s"]) == 3
    assert bench._pieces([5, 0, 7, 1], 3) == [[(0, 0, 4)], [(0, 4, 5), (2, 0, 3)], [(2, 3, 7), (3, 0, 1)]]


def test_request_counters_give_bytes_without_calibration(tmp_path):
    """Reads: 32/64/128-byte requests times their size; writes: 32/64-byte;
    the FETCH_SIZE formula reads 128-byte requests only through TCC_BUBBLE,
    so with TCC_BUBBLE at zero it reports half of all-128-byte reads.
    Rows of one dispatch from several counter instances are summed."""
    import json as _json
    copy = "void at::native::elementwise_copy_kernel(...)"
    win = "gro::(anonymous namespace)::k_accumulate_window(gro::WindowLaunch)"
    rd, wr = tmp_path / "rd.csv", tmp_path / "wr.csv"
    mib = 1 << 20
    rows_rd, rows_wr = [], []
    for d in range(3):  # copy: 1 MiB each way as 128-byte reads and 64-byte writes, two instances each
        for half in (0, 1):
            rows_rd += [(d, copy, "TCC_EA0_RDREQ", mib // 256), (d, copy, "TCC_EA0_RDREQ_32B", 0),
                        (d, copy, "TCC_EA0_RDREQ_64B", 0), (d, copy, "TCC_EA0_RDREQ_128B", mib // 256)]
            rows_wr += [(d, copy, "TCC_EA0_WRREQ", mib // 128), (d, copy, "TCC_EA0_WRREQ_64B", mib // 128),
                        (d, copy, "TCC_BUBBLE", 0)]
    rows_rd += [(7, win, "TCC_EA0_RDREQ", 110), (7, win, "TCC_EA0_RDREQ_32B", 4),
                (7, win, "TCC_EA0_RDREQ_64B", 6), (7, win, "TCC_EA0_RDREQ_128B", 100)]
    rows_wr += [(7, win, "TCC_EA0_WRREQ", 50), (7, win, "TCC_EA0_WRREQ_64B", 40), (7, win, "TCC_BUBBLE", 0)]
    for path, rows in ((rd, rows_rd), (wr, rows_wr)):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=COLS)
            w.writeheader()
            for i, (d, k, c, val) in enumerate(rows):
                w.writerow({"Correlation_Id": i, "Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c,
                            "Counter_Value": val})
    r = P.requests(mib, [str(rd), str(wr)])
    c = r["kernels"]["copy"]
    assert c["read_counted_over_known"] == pytest.approx(1.0) and c["write_counted_over_known"] == pytest.approx(1.0)
    assert c["fetch_size_formula_bytes"] == pytest.approx(mib / 2)
    k = r["kernels"]["k_accumulate_window"]
    assert k["read_bytes_per_launch"] == 32 * 4 + 64 * 6 + 128 * 100
    assert k["write_bytes_per_launch"] == 32 * 10 + 64 * 40
    assert k["fetch_size_formula_bytes"] == 32 * 4 + 64 * 106
    _json.dumps(r)


def test_probe_kernels_keep_their_template_arguments():
    assert P.short_name("void (anonymous namespace)::probe_window<16, 8>((anonymous namespace)::Streams)") == \
        "probe_window<16, 8>"
    assert P.short_name("void (anonymous namespace)::probe_adamw<4>((anonymous namespace)::Streams, long)") == \
        "probe_adamw<4>"
