"""Summaries of rocprofv3 runs of bench.py for the profiles/ directory.

    python -m paged_kv_cache_163_amd.profiling stats   TRACE_DIR  OUT.md  "COMMAND"
    python -m paged_kv_cache_163_amd.profiling counters PMC_DIR KERNEL WORKLOAD OUT.md "COMMAND"
    python -m paged_kv_cache_163_amd.profiling traffic FETCH_DIR WRITE_DIR CAL_FETCH_DIR \
        CAL_WRITE_DIR KERNEL WORKLOAD OUT.json OUT.md "COMMANDS"

``stats`` condenses a ``rocprofv3 --kernel-trace --stats`` run (the
``*_kernel_stats.csv`` it writes) into a markdown table; ``counters`` does the
same for the per-dispatch values of one kernel in a ``--pmc`` run.

``traffic`` turns two ``rocprofv3 --pmc`` runs of the benchmark (FETCH_SIZE,
then WRITE_SIZE, in KiB per dispatch) into HBM bytes per launch of KERNEL.
Each counter is scaled by what it reads for a plain device copy of known size
(``bench.py --copy-calibration``: 1 GiB read and 1 GiB written per launch),
so the figure is in real bytes whatever unit or XCD coverage the counter has.
The JSON record carries a hash of the kernel's sources; bench.py only
reports it while the sources are unchanged.
"""

from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys

COPY_BYTES = 1 << 30


def _csv(directory: str, suffix: str) -> list[dict]:
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


TAIL_CALLS = 100   # the benchmark's timed launches come last in its run


def _tail_avg_us(trace_dir: str) -> dict:
    """Average duration (us) of each kernel's last TAIL_CALLS dispatches in
    the kernel trace: the steady state after the run's warm-up launches."""
    try:
        rows = _csv(trace_dir, "kernel_trace.csv")
    except FileNotFoundError:
        return {}
    per = {}
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, d in per.items():
        tail = [ns for _, ns in sorted(d)[-TAIL_CALLS:]]
        out[name] = sum(tail) / len(tail) / 1e3
    return out


def kernel_stats_md(trace_dir: str, command: str) -> str:
    rows = _csv(trace_dir, "kernel_stats.csv")
    tail = _tail_avg_us(trace_dir)
    lines = [f"Command: `{command}`", "",
             f"| kernel | calls | avg us | min us | max us | share % | avg us, last {TAIL_CALLS} calls |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        t = tail.get(r["Name"])
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} | {'' if t is None else f'{t:.2f}'} |")
    return "\n".join(lines) + "\n"


def _per_dispatch(directory: str, counter: str, kernel_prefix: str) -> list[float]:
    rows = _csv(directory, "counter_collection.csv")
    return [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and r["Kernel_Name"].startswith(kernel_prefix)]


def traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, kernel):
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    write = _per_dispatch(write_dir, "WRITE_SIZE", kernel)
    cal_f = _per_dispatch(cal_fetch_dir, "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    cal_w = _per_dispatch(cal_write_dir, "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    f_scale = COPY_BYTES / (statistics.median(cal_f) * 1024)   # bytes per KiB read
    w_scale = COPY_BYTES / (statistics.median(cal_w) * 1024)
    f_bytes = statistics.median(fetch) * 1024 * f_scale
    w_bytes = statistics.median(write) * 1024 * w_scale
    return {
        "fetch_kib_per_dispatch": statistics.median(fetch),
        "write_kib_per_dispatch": statistics.median(write),
        "copy_fetch_kib": statistics.median(cal_f),
        "copy_write_kib": statistics.median(cal_w),
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_read_bytes_per_launch": f_bytes,
        "hbm_write_bytes_per_launch": w_bytes,
        "hbm_bytes_per_launch": f_bytes + w_bytes,
        "dispatches": len(fetch),
    }


def counters_md(run_dir: str, kernel: str, workload: str, command: str) -> str:
    """Per-dispatch counter values of KERNEL (median over its dispatches, in
    millions) from a ``rocprofv3 --pmc`` run."""
    rows = [r for r in _csv(run_dir, "counter_collection.csv")
            if r["Kernel_Name"].startswith(kernel)]
    by: dict[str, dict[str, float]] = {}
    for r in rows:  # one row per (dispatch, counter)
        d = by.setdefault(r["Counter_Name"], {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    lines = [f"Command: `{command}`", "",
             f"Kernel `{kernel}`, workload `{workload}`; counter sums per dispatch (median over "
             f"{len(next(iter(by.values()), {}))} dispatches), millions.", "",
             "| counter | per dispatch (M) |", "|---|---|"]
    for name in sorted(by):
        lines.append(f"| {name} | {statistics.median(by[name].values()) / 1e6:.2f} |")
    return "\n".join(lines) + "\n"


def main(argv):
    if argv[0] == "counters":
        run_dir, kernel, workload, out_md, command = argv[1:6]
        with open(out_md, "w") as f:
            f.write(counters_md(run_dir, kernel, workload, command))
        return
    if argv[0] == "stats":
        trace_dir, out_md, command = argv[1:4]
        with open(out_md, "w") as f:
            f.write(kernel_stats_md(trace_dir, command))
        return
    if argv[0] == "traffic":
        fd, wd, cfd, cwd, kernel, workload, out_json, out_md, commands = argv[1:10]
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        rec = traffic(fd, wd, cfd, cwd, kernel)
        rec.update({"kernel": kernel, "workload": workload,
                    "kernel_source_hash": bench.source_hash(kernel)})
        with open(out_json, "w") as f:
            json.dump(rec, f, indent=1)
        with open(out_md, "w") as f:
            f.write(f"Commands: {commands}\n\n")
            f.write(f"Kernel `{kernel}`, workload `{workload}`.\n\n")
            f.write("| quantity | value |\n|---|---|\n")
            for k in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "copy_fetch_kib",
                      "copy_write_kib", "fetch_scale", "write_scale",
                      "hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch",
                      "hbm_bytes_per_launch", "dispatches"):
                f.write(f"| {k} | {rec[k]:.6g} |\n")
        return
    raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
