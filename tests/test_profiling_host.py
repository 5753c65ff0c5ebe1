"""Host tests of the rocprofv3 summary helpers and bench.py's argument
handling (no GPU needed).  The CSV rows below are hand-made fixtures in
rocprofv3's column layout, not measurements."""
import csv
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
