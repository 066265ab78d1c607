"""The measurement harness on the CPU: bench.py's multi-GPU refusal, the
counter records it trusts only while the kernel sources are unchanged, and the
rocprofv3 summaries of paged_kv_cache_163_amd/profiling.py on synthetic CSVs, and
the power sampler on a stand-in amd-smi."""

import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_traffic_record_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    import bench
    for rel in bench.KERNEL_SOURCES["decode_mfma_kernel"]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"workload": "llama70b", "hbm_bytes_per_launch": 123.0,
           "kernel_source_hash": bench.source_hash("decode_mfma_kernel")}
    path = tmp_path / "profiles" / "decode_mfma_llama70b_traffic.json"
    path.write_text(json.dumps(rec))
    assert bench.traffic_entry("llama70b") == 123.0
    assert bench.traffic_entry("sweep_b16_d64") is None          # no record for it
    src = tmp_path / bench.KERNEL_SOURCES["decode_mfma_kernel"][0]
    src.write_text(src.read_text() + "\n// changed\n")          # the kernel changed since
    assert bench.traffic_entry("llama70b") is None


def _write_counters(path, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(fields, r)))


def test_traffic_scales_counters_by_the_copy_calibration(tmp_path):
    from paged_kv_cache_163_amd import profiling as P
    for d in ("f", "w", "cf", "cw"):
        (tmp_path / d).mkdir()
    # kernel: FETCH 1000 / 1200 / 1100 KiB per dispatch (median 1100), WRITE 50 KiB
    _write_counters(tmp_path / "f" / "x_counter_collection.csv",
                    [(i, "decode_mfma_kernel", "FETCH_SIZE", v)
                     for i, v in enumerate((1000, 1200, 1100))])
    _write_counters(tmp_path / "w" / "x_counter_collection.csv",
                    [(i, "decode_mfma_kernel", "WRITE_SIZE", 50) for i in range(3)])
    # the 1 GiB copy reads as half its size on FETCH_SIZE and whole on WRITE_SIZE
    _write_counters(tmp_path / "cf" / "x_counter_collection.csv",
                    [(0, "__amd_rocclr_copyBuffer", "FETCH_SIZE", (1 << 20) / 2)])
    _write_counters(tmp_path / "cw" / "x_counter_collection.csv",
                    [(0, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1 << 20)])
    rec = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                    str(tmp_path / "cw"), "decode_mfma_kernel")
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == pytest.approx(1100 * 1024 * 2)
    assert rec["hbm_write_bytes_per_launch"] == pytest.approx(50 * 1024)
    assert rec["dispatches"] == 3


def test_kernel_stats_add_the_steady_state_of_the_last_calls(tmp_path):
    from paged_kv_cache_163_amd import profiling as P
    with open(tmp_path / "x_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow(["k", 150, 0, 5000.0, 100.0, 1000.0, 9000.0])
    # 50 slow warm-up calls of 9 us, then 100 of 1 us, written out of order
    calls = [(1000 * i, 9000) for i in range(50)] + [(1000 * i, 1000) for i in range(50, 150)]
    with open(tmp_path / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for start, dur in reversed(calls):
            w.writerow(["k", start, start + dur])
    md = P.kernel_stats_md(str(tmp_path), "cmd")
    assert "| k | 150 | 5.00 | 1.00 | 9.00 | 100.00 | 1.00 |" in md


def test_counter_summary_sums_per_dispatch_and_takes_the_median(tmp_path):
    from paged_kv_cache_163_amd import profiling as P
    rows = []
    for disp, vals in ((1, (1e6, 2e6)), (2, (3e6, 4e6)), (3, (5e6, 6e6))):
        for v in vals:   # two rows per dispatch (e.g. two XCD shares), summed
            rows.append((disp, "prefill_mfma_kernel", "SQ_WAVE_CYCLES", v))
    rows.append((4, "other_kernel", "SQ_WAVE_CYCLES", 1e9))
    _write_counters(tmp_path / "x_counter_collection.csv", rows)
    md = P.counters_md(str(tmp_path), "prefill_mfma_kernel", "w", "cmd")
    assert "| SQ_WAVE_CYCLES | 7.00 |" in md        # per-dispatch sums 3, 7, 11 -> median 7
    assert "median over 3 dispatches" in md


def test_cpu_baseline_summary_takes_the_median_run_and_measured_cores():
    """cpu_baseline: three runs, the median rate reported, `cores` = process
    CPU time over wall time (rounded, at least 1), the runs and BLAS listed."""
    import bench
    runs = [(30, 2.0, 2.0), (10, 2.0, 2.1), (20, 2.0, 1.9)]       # (units, wall, cpu)
    res = bench._baseline_summary(runs, 1.0, "u/s", "sample")
    assert res["value"] == 10.0 and res["runs"] == [5.0, 10.0, 15.0]
    assert res["cores"] == 1 and res["cores_used"] == 1.0
    res = bench._baseline_summary([(8, 1.0, 3.6)], 1.0, "u/s", "sample")
    assert res["cores"] == 4
    assert {"vendor", "threads"} <= set(res["blas"]) and res["affinity_cpus"] >= 1
    assert res["kind"] == "oracle"


class _FakeCuda:
    @staticmethod
    def synchronize():
        pass


class _FakeTorch:
    cuda = _FakeCuda()


def test_power_sampler_reads_amd_smi_json(tmp_path, monkeypatch):
    """bench.sample_power runs the step while a thread reads `amd-smi metric
    -p -c --json`: medians of socket power and of the mean graphics clock over
    the samples taken while busy; None without amd-smi."""
    import bench
    fake = tmp_path / "amd-smi"
    reading = {"gpu_data": [{"gpu": 0,
                             "power": {"socket_power": {"value": 1390, "unit": "W"}},
                             "clock": {"gfx_0": {"clk": {"value": 2200, "unit": "MHz"}},
                                       "gfx_1": {"clk": {"value": 2300, "unit": "MHz"}},
                                       "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}}}]}
    fake.write_text("#!/bin/sh\ncat <<'JSON'\n" + json.dumps(reading) + "\nJSON\n")
    fake.chmod(0o755)
    monkeypatch.setenv("PATH", str(tmp_path) + os.pathsep + os.environ.get("PATH", ""))
    calls = []
    res = bench.sample_power(_FakeTorch, lambda i: calls.append(i), 1.0)
    assert res is not None and calls
    assert res["socket_power_w"] == 1390.0
    assert res["gfx_clock_mhz"] == 2250.0          # mean of the graphics clocks only
    assert res["samples"] >= 1
    monkeypatch.setenv("PATH", str(tmp_path / "nowhere"))
    assert bench.sample_power(_FakeTorch, lambda i: None, 1.0) is None
    assert bench.sample_power(_FakeTorch, lambda i: None, 0.0) is None
