"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama70b]

A step is one pass of the whole decode path over one synthetic batch:
copy-on-write block copies of the batch (if any), KV append of the batch's new
tokens, then paged decode attention.  The decode gets the batch's
longest-first order, computed once before timing: every step adds one token to
every sequence, so the order holds from step to step (--rank-in-kernel makes
each work-group rank the batch instead).  The append is its own launch
(pa_kv_append) unless --fused-append moves it into the decode launch
(pa_decode_append), which measured ~2 us slower per step on the 70B batch.  Inputs are generated on the host,
uploaded, and resident in HBM before timing starts.  The KV pools are
replicated ``--rotate`` times and step i uses copy i mod rotate, so a step
never finds the previous step's blocks in the 256 MB MALL / L2.

Prints ONE JSON line.  ``value`` is live-KV GB/s of the whole step (live KV
bytes the decode must read / step time).  ``roofline`` describes the dominant
kernel (the decode kernel): achieved = live KV bytes per launch / its average
launch time, timed with HIP events around each decode call on the stream the
library launches on.  The events skip the system-scope cache fence, so timing
adds no idle gap between launches.  ``cpu_baseline`` times the CPU oracle on a bounded
sample of the same batch.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "paged decode attention: achieved KV GB/s (% of HBM peak) and seqs/sec, 1 GPU"
# Sources each profiled kernel is built from: a stored counter record is used
# only while their hash still matches.
_CSRC = "paged_kv_cache_163_amd/csrc/"
KERNEL_SOURCES = {
    "decode_mfma_kernel": [_CSRC + f for f in ("decode_mfma.hip", "decode_mfma.h", "mfma_step.h",
                                               "pa_internal.h")],
    "prefill_mfma_kernel": [_CSRC + f for f in ("prefill_mfma.hip", "row_tiles.h", "mfma_step.h",
                                                "pa_internal.h")],
    "shared_prefix_kernel": [_CSRC + f for f in ("shared_prefix.hip", "decode_mfma.h",
                                                 "row_tiles.h", "mfma_step.h", "pa_internal.h")],
    "decode_reduce_kernel": [_CSRC + f for f in ("decode_reduce.hip", "pa_internal.h")],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama70b",
                    help="llama70b | shared_prefix | long_context | sweep_b{16,32,64}_d{64,128} "
                         "| prefill_llama70b | prefill_chunked (one pa_prefill launch per step) "
                         "| swap_llama70b (block swap to pinned host memory and back) "
                         "| layered_llama70b (8 layers of a layered pool per launch)")
    ap.add_argument("--rotate", type=int, default=4, help="KV pool copies cycled over steps")
    ap.add_argument("--partition", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--kernel", default="auto", choices=["auto", "mfma", "valu"])
    ap.add_argument("--fused-append", action="store_true",
                    help="append inside the decode launch (pa_decode_append)")
    ap.add_argument("--rank-in-kernel", action="store_true",
                    help="let every decode work-group rank the batch (pa_decode) instead of "
                         "passing the longest-first order the step keeps (pa_decode_ordered)")
    ap.add_argument("--index-order", action="store_true",
                    help="shared_prefix: the tails in index order (pa_decode_shared_prefix) "
                         "instead of longest first (pa_decode_shared_prefix_ordered)")
    ap.add_argument("--plain-decode", action="store_true",
                    help="shared_prefix: time pa_decode instead of the shared-prefix decode "
                         "(pa_decode_shared_prefix)")
    ap.add_argument("--prefix-partition", type=int, default=0,
                    help="shared_prefix: keys per prefix partition (0 = library's choice)")
    ap.add_argument("--prefill-warmup-ms", type=float, default=300.0,
                    help="prefill workloads: warm up for at least this long (clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time for cpu_baseline, split over three runs")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="decode workloads: skip timing the other configs after the headline")
    ap.add_argument("--power-seconds", type=float, default=0.0,
                    help="after the measurement, repeat the step for this long while sampling "
                         "the board's power and graphics clocks (amd-smi); 0 = off")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def source_hash(kernel: str = "decode_mfma_kernel") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry(workload: str, kernel: str = "decode_mfma_kernel"):
    """HBM bytes per launch of `kernel` on `workload` from committed rocprofv3
    counter runs, or None when absent or taken on a different version of the
    kernel's sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel[:-len('_kernel')]}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != source_hash(kernel) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def sample_power(torch, step, seconds):
    """Repeat `step` for `seconds` while another thread reads the board's
    socket power and graphics clocks through `amd-smi metric` every ~0.3 s.
    Reports the medians of the samples taken while the GPU was busy (the
    first and last samples can straddle the loop's edges), or None when
    amd-smi is not available."""
    import shutil
    import subprocess
    import threading
    if seconds <= 0 or shutil.which("amd-smi") is None:
        return None
    samples, stop = [], threading.Event()

    def reader():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", "0", "--json"],
                                   capture_output=True, text=True, timeout=20)
                d = json.loads(r.stdout)
                d = d[0] if isinstance(d, list) else d
                d = d["gpu_data"][0] if "gpu_data" in d else d
                watts = float(d["power"]["socket_power"]["value"])
                clks = [float(v["clk"]["value"]) for k, v in d["clock"].items()
                        if k.startswith("gfx_") and isinstance(v, dict)]
                samples.append((watts, sum(clks) / len(clks) if clks else None))
            except Exception:  # a malformed or missing reading is skipped
                pass
            stop.wait(0.3)

    th = threading.Thread(target=reader, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step(n)
            n += 1
        torch.cuda.synchronize()
    stop.set()
    th.join()
    busy = samples[1:-1] if len(samples) > 2 else samples
    if not busy:
        return None
    watts = sorted(w for w, _ in busy)
    clks = sorted(c for _, c in busy if c is not None)
    return {"socket_power_w": watts[len(watts) // 2],
            "gfx_clock_mhz": round(clks[len(clks) // 2], 1) if clks else None,
            "samples": len(busy), "seconds": seconds, "source": "amd-smi metric -p -c"}


class HipTimer:
    """HIP timing events on torch's own HIP runtime, recorded without the
    system-scope fence (hipEventDisableSystemFence).  A default event's fence
    writes back and invalidates the caches and left ~5 us of idle GPU per
    record between launches; these only take timestamps."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self._c = ctypes
        self._hip = ctypes.CDLL(path)  # already mapped: the same runtime torch uses
        self._events = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def event(self):
        e = self._c.c_void_p()
        self._check(self._hip.hipEventCreateWithFlags(self._c.byref(e),
                                                      self._c.c_uint(self.DISABLE_SYSTEM_FENCE)),
                    "hipEventCreateWithFlags")
        self._events.append(e)
        return e

    def record(self, e, stream):
        self._check(self._hip.hipEventRecord(e, self._c.c_void_p(stream.cuda_stream)),
                    "hipEventRecord")

    def elapsed_ms(self, a, b):
        ms = self._c.c_float()
        self._check(self._hip.hipEventElapsedTime(self._c.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def close(self):
        for e in self._events:
            self._hip.hipEventDestroy(e)
        self._events = []


def blas_info() -> dict:
    """numpy's BLAS as threadpoolctl reports it: vendor, version, threads."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # threadpoolctl missing: nothing known
        blas = []
    if not blas:
        return {"vendor": "unknown", "version": None, "threads": 1}
    b = blas[0]
    return {"vendor": b.get("internal_api", "unknown"), "version": b.get("version"),
            "threads": int(b.get("num_threads", 1))}


def host_cpus() -> int:
    """CPUs this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _timed_runs(one_unit, seconds: float, runs: int = 3):
    """Call one_unit() (returning units of work done) until seconds/runs pass,
    `runs` times.  Returns [(units, wall_s, cpu_s)] per run; cpu_s is the
    process CPU time over the run, so cpu_s / wall_s is the cores it used."""
    out = []
    for _ in range(runs):
        units = 0
        t0, c0 = time.perf_counter(), time.process_time()
        while time.perf_counter() - t0 < seconds / runs:
            units += one_unit()
        out.append((units, time.perf_counter() - t0, time.process_time() - c0))
    return out


def _baseline_summary(runs, unit_scale: float, unit: str, sample: str) -> dict:
    rates = sorted(u * unit_scale / w for u, w, _ in runs)
    med = rates[len(rates) // 2]
    cores_used = sum(c for _, _, c in runs) / sum(w for _, w, _ in runs)
    info = blas_info()
    return {
        "value": round(med, 9),
        "unit": unit,
        "cores": max(1, int(round(cores_used))),
        "kind": "oracle",
        "sample": sample,
        "runs": [round(r, 9) for r in rates],
        "cores_used": round(cores_used, 2),
        "blas": info,
        "affinity_cpus": host_cpus(),
        "logical_cpus": os.cpu_count(),
    }


def cpu_baseline(w, seconds: float):
    """The oracle, as it stands, on whole-batch sequences: three runs of
    seconds/3 each (median reported), numpy's BLAS allowed every CPU of this
    process's affinity mask; `cores` is the CPU time over wall time it took."""
    import numpy as np

    import oracle
    order = np.random.default_rng(123).permutation(w.num_seqs)
    state = {"i": 0, "seqs": 0}
    per_tok = 2 * w.kv_heads * w.head_dim * w.elem_bytes

    def one():
        s = int(order[state["i"] % w.num_seqs])
        state["i"] += 1
        state["seqs"] += 1
        oracle.paged_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.scale,
                            w.block_size, seqs=[s])
        return int(w.seq_lens[s]) * per_tok

    limits = None
    try:
        from threadpoolctl import threadpool_limits
        limits = threadpool_limits(limits=host_cpus(), user_api="blas")
    except Exception:  # threadpoolctl missing: numpy's default thread count
        pass
    try:
        runs = _timed_runs(one, seconds)
    finally:
        if limits is not None:
            limits.restore_original_limits()
    total_wall = sum(wall for _, wall, _ in runs)
    res = _baseline_summary(
        runs, 1e-9, "GB/s",
        f"{state['seqs']} sequences of the {w.name} batch (random order, seed 123) in 3 runs "
        f"of {seconds / 3:.1f} s, one process, numpy float64, median run reported")
    res["seqs_per_s"] = round(state["seqs"] / total_wall, 3)
    return res


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, vendor figure
PREFILL_METRIC = "paged chunked prefill attention: achieved TFLOP/s (% of bf16 MFMA peak), 1 GPU"


def prefill_cpu_baseline(w, seconds: float):
    """The oracle, as it stands, on query rows of the batch (three runs of
    seconds/3, median reported), BLAS over this process's CPUs."""
    import numpy as np

    import oracle
    from paged_kv_cache_163_amd import workloads as W
    order = np.random.default_rng(123).permutation(w.num_queries)
    starts = w.query_start
    state = {"i": 0}

    def one():
        r = int(order[state["i"] % w.num_queries])
        state["i"] += 1
        oracle.paged_prefill(w.q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.query_lens,
                             w.scale, w.block_size, rows=[r])
        s = int(np.searchsorted(starts, r, side="right")) - 1
        pos = int(w.seq_lens[s] - w.query_lens[s] + (r - starts[s]))
        return W.prefill_flops([pos + 1], [1], w.num_heads, w.head_dim)

    limits = None
    try:
        from threadpoolctl import threadpool_limits
        limits = threadpool_limits(limits=host_cpus(), user_api="blas")
    except Exception:  # threadpoolctl missing: numpy's default thread count
        pass
    try:
        runs = _timed_runs(one, seconds)
    finally:
        if limits is not None:
            limits.restore_original_limits()
    return _baseline_summary(
        runs, 1e-12, "TFLOP/s",
        f"{state['i']} query rows of the {w.name} batch (random order, seed 123, each with its "
        f"sequence's gather) in 3 runs of {seconds / 3:.1f} s, one process, numpy float64, "
        "median run reported")


def prefill_timed(np, torch, W, pa, dev, name, steps, warmup, warmup_ms, rotate):
    """Steady-state pa_prefill timing of workload `name`: (workload, mean
    launch ms, launches made before the timed region, step function)."""
    w = W.PREFILL_WORKLOADS[name]()

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    pools = [(to_dev(w.k_cache), to_dev(w.v_cache)) for _ in range(max(1, rotate))]
    q, bt, lens, qs = to_dev(w.q), to_dev(w.block_tables), to_dev(w.seq_lens), to_dev(w.query_start)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(i):
        kc, vc = pools[i % len(pools)]
        pa.prefill(q, kc, vc, bt, lens, qs, w.scale, max_query_len=w.max_query_len, out=out)

    # The matrix-core prefill is clock-bound, and the clock ramps up over tens
    # of milliseconds of load after an idle gap (a 50-launch run measured
    # 392 us for its first timed launch, 334 us for its last).  So the warmup
    # runs at least `warmup_ms` of launches, and the timed region starts right
    # after the synchronize, with its events made beforehand.
    timer = HipTimer()
    t_start, t_end = timer.event(), timer.event()
    step(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step(1)
    torch.cuda.synchronize()
    one_ms = max((time.perf_counter() - t0) * 1e3, 1e-3)
    warm = max(warmup, int(warmup_ms / one_ms) + 1)
    for i in range(warm):
        step(2 + i)
    torch.cuda.synchronize()
    timer.record(t_start, stream)
    for i in range(steps):
        step(2 + warm + i)
    timer.record(t_end, stream)
    torch.cuda.synchronize()
    step_ms = timer.elapsed_ms(t_start, t_end) / steps
    timer.close()
    return w, step_ms, warm + 2, step


def prefill_line(W, w, step_ms):
    """TFLOP/s, roofline fraction and launch time of one prefill measurement."""
    flops = W.prefill_flops(w.seq_lens, w.query_lens, w.num_heads, w.head_dim)
    tflops = flops / (step_ms * 1e-3) / 1e12
    return {"workload": w.name, "launch_us": round(step_ms * 1e3, 2),
            "tflops": round(tflops, 2), "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "queries_per_s": round(w.num_queries / (step_ms * 1e-3), 1)}


def prefill_main(args, np, torch, W, pa, dev):
    """One step = one pa_prefill launch over the whole batch of chunks."""
    w, step_ms, launched, step = prefill_timed(np, torch, W, pa, dev, args.workload, args.steps,
                                               args.warmup, args.prefill_warmup_ms, args.rotate)
    flops = W.prefill_flops(w.seq_lens, w.query_lens, w.num_heads, w.head_dim)
    tflops = flops / (step_ms * 1e-3) / 1e12
    kv_bytes = W.decode_kv_bytes(w.seq_lens, w.kv_heads, w.head_dim, w.elem_bytes)
    line = {
        "metric": PREFILL_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs,
            "num_queries": w.num_queries,
            "num_heads": w.num_heads,
            "kv_heads": w.kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "mean_seq_len": round(float(w.seq_lens.mean()), 2),
            "mean_chunk": round(float(w.query_lens.mean()), 2),
            "pool_rotation": max(1, args.rotate),
            "warmup_launches": launched,
            "parallelism": "single GPU",
        },
        "flops_per_step": flops,
        "tokens_per_s": round(w.num_queries / (step_ms * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_entry(w.name, "prefill_mfma_kernel"),
            "kernel": "prefill_mfma_kernel",
            "flops_per_launch": flops,
            "avg_launch_ms": round(step_ms, 5),
        },
        "cpu_baseline": None,
    }
    if args.power_seconds > 0:
        line["power"] = sample_power(torch, lambda i: step(i), args.power_seconds)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


SWAP_METRIC = "KV block swap for preemption: GB/s over the host link (device->host, host->device), 1 GPU"
HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, per direction


def swap_main(args, np, torch, W, pa, dev):
    """Preempt 32 sequences of 850 tokens (the pages' 600 + 250 request, 54
    blocks each) on the 70B layer shape: their blocks go to a pinned host pool
    and come back into other device blocks.  Each direction is one
    pa_swap_blocks launch, timed separately."""
    rng = np.random.default_rng(0)
    seqs, blocks_per_seq = 32, 54
    n = seqs * blocks_per_seq
    shape = (8, 16, 128)
    dev_blocks = 2 * n + 64
    dk = torch.empty((dev_blocks,) + shape, dtype=torch.bfloat16, device=dev)
    dv = torch.empty_like(dk)
    g = torch.Generator(device=dev).manual_seed(0)
    dk.normal_(generator=g)
    dv.normal_(generator=g)
    hk = torch.empty((n,) + shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    perm = rng.permutation(dev_blocks)
    out_pairs = torch.from_numpy(np.stack([perm[:n], rng.permutation(n)], 1).astype(np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), perm[n:2 * n]], 1).astype(np.int64)).to(dev)
    bytes_moved = 2 * n * int(np.prod(shape)) * 2
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        timer = HipTimer()
        a, b = timer.event(), timer.event()
        timer.record(a, stream)
        for _ in range(args.steps):
            fn()
        timer.record(b, stream)
        torch.cuda.synchronize()
        ms = timer.elapsed_ms(a, b) / args.steps
        timer.close()
        return ms

    out_ms = timed(lambda: pa.swap_blocks(hk, hv, dk, dv, out_pairs))
    in_ms = timed(lambda: pa.swap_blocks(dk, dv, hk, hv, in_pairs))
    # context: one contiguous DMA copy of the same bytes each way
    flat_d = torch.empty(bytes_moved // 2, dtype=torch.bfloat16, device=dev)
    flat_h = torch.empty(bytes_moved // 2, dtype=torch.bfloat16, pin_memory=True)
    dma_out_ms = timed(lambda: flat_h.copy_(flat_d, non_blocking=True))
    dma_in_ms = timed(lambda: flat_d.copy_(flat_h, non_blocking=True))
    out_gbs = bytes_moved / (out_ms * 1e-3) / 1e9
    in_gbs = bytes_moved / (in_ms * 1e-3) / 1e9
    total_gbs = 2 * bytes_moved / ((out_ms + in_ms) * 1e-3) / 1e9
    line = {
        "metric": SWAP_METRIC,
        "value": round(total_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(out_ms + in_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swap_llama70b", "preempted_seqs": seqs,
                   "blocks_per_seq": blocks_per_seq, "blocks": n, "kv_heads": 8,
                   "block_size": 16, "head_dim": 128, "parallelism": "single GPU"},
        "bytes_per_direction": bytes_moved,
        "device_to_host": {"ms": round(out_ms, 5), "GBps": round(out_gbs, 2)},
        "host_to_device": {"ms": round(in_ms, 5), "GBps": round(in_gbs, 2)},
        "contiguous_dma_copy": {"device_to_host_GBps": round(bytes_moved / (dma_out_ms * 1e-3) / 1e9, 2),
                                "host_to_device_GBps": round(bytes_moved / (dma_in_ms * 1e-3) / 1e9, 2)},
        "roofline": {"bound": "host_link", "achieved": round(total_gbs, 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(total_gbs / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                     "kernel": "move_blocks_kernel", "bytes_per_launch": bytes_moved,
                     "avg_launch_ms": round((out_ms + in_ms) / 2, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def layered_main(args, np, torch, W, pa, dev, layers=8):
    """The 70B-shaped decode batch over a layered pool of `layers` layers
    ([num_blocks, 2, layers, 8, 16, 128] bf16, filled on the device): all
    layers in one pa_decode_layered launch, against one launch per layer."""
    w = W.llama70b(append=False)
    shape = (w.num_blocks, 2, layers, w.kv_heads, w.block_size, w.head_dim)
    pool = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev).manual_seed(0)
    pool.normal_(generator=g)
    q = torch.empty((layers,) + w.q.shape, dtype=torch.bfloat16, device=dev).normal_(generator=g)
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty_like(q)
    plan = pa.decode_plan(w.num_seqs, w.num_heads, w.kv_heads, w.head_dim, w.block_size,
                          w.max_seq_len, 0, torch.bfloat16, "mfma")
    ws = torch.empty(max(plan.workspace_bytes * layers, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def all_layers():
        pa.decode_layered(q, pool, bt, lens, w.scale, max_seq_len=w.max_seq_len, out=out,
                          workspace=ws)

    def per_layer():
        for layer in range(layers):
            pa.decode_layered(q[layer:layer + 1], pool, bt, lens, w.scale, first_layer=layer,
                              max_seq_len=w.max_seq_len, out=out[layer:layer + 1], workspace=ws)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        timer = HipTimer()
        a, b = timer.event(), timer.event()
        timer.record(a, stream)
        for _ in range(args.steps):
            fn()
        timer.record(b, stream)
        torch.cuda.synchronize()
        ms = timer.elapsed_ms(a, b) / args.steps
        timer.close()
        return ms

    one_ms = timed(all_layers)
    each_ms = timed(per_layer)
    kv_bytes = layers * W.decode_kv_bytes(w.seq_lens, w.kv_heads, w.head_dim, w.elem_bytes)
    gbs = kv_bytes / (one_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC + " (layered pool, all layers per launch)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(one_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "layered_llama70b", "layers": layers, "num_seqs": w.num_seqs,
                   "num_heads": w.num_heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "partition_size": plan.partition_size, "parallelism": "single GPU"},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "one_launch_per_layer": {"ms": round(each_ms, 5),
                                 "GBps": round(kv_bytes / (each_ms * 1e-3) / 1e9, 2)},
        "kv_bytes_per_step": kv_bytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_mfma_kernel (layered)", "bytes_per_launch": kv_bytes,
                     "avg_launch_ms": round(one_ms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


class DecodeRun:
    """One decode workload resident on the device, ready to step.

    A step is the workload's copy-on-write copies, its KV append, then the
    decode: pa_decode_ordered with the batch's longest-first order (computed
    once: every step adds one token to every sequence, so the order holds),
    pa_decode_shared_prefix on the shared-prefix batch, pa_decode_append with
    `fused`, pa_decode with `rank_in_kernel`.  The K/V pools are replicated
    `rotate` times and step i uses copy i mod rotate, so a step never finds
    the previous step's blocks in the 256 MB MALL / L2.  `host_fill` uploads
    the workload's seeded pools (the parity tests' bytes); otherwise the pools
    are filled with N(0,1) on the device (timing only)."""

    def __init__(self, np, torch, W, pa, dev, name, *, rotate=4, partition=0, kernel="auto",
                 fused=False, rank_in_kernel=False, plain_decode=False, prefix_partition=0,
                 host_fill=True, index_order=False):
        self.np, self.torch, self.pa, self.W = np, torch, pa, W
        w = self.w = W.make(name, fill=host_fill)
        self.partition, self.kernel, self.prefix_partition = partition, kernel, prefix_partition

        def to_dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        if host_fill:
            self.pools = [(to_dev(w.k_cache), to_dev(w.v_cache)) for _ in range(max(1, rotate))]
        else:
            g = torch.Generator(device=dev).manual_seed(0)
            dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
            self.pools = []
            for _ in range(max(1, rotate)):
                k = torch.empty(w.k_cache.shape, dtype=dt, device=dev).normal_(generator=g)
                self.pools.append((k, torch.empty_like(k).normal_(generator=g)))
        self.q = to_dev(w.q)
        self.bt, self.lens = to_dev(w.block_tables), to_dev(w.seq_lens)
        self.k_new, self.v_new = to_dev(w.k_new), to_dev(w.v_new)
        self.slots = to_dev(w.slot_mapping)
        self.fk, self.fv, self.fslots = (to_dev(a) for a in W.per_sequence_append(w))
        self.fused = w.slot_mapping.shape[0] > 0 and fused
        self.pairs = to_dev(w.cow_pairs)
        self.out = torch.empty_like(self.q)
        self.plan = pa.decode_plan(w.num_seqs, w.num_heads, w.kv_heads, w.head_dim,
                                   w.block_size, w.max_seq_len, partition, self.q.dtype, kernel)
        ws_bytes = self.plan.workspace_bytes
        # Shared-prefix batch: every table starts with the same prefix blocks,
        # so the shared-prefix decode attends them once for the whole group.
        self.shared = ("prefix_blocks" in w.meta and not plain_decode and not self.fused
                       and kernel in ("auto", "mfma"))
        if self.shared:
            self.groups = ([0, w.num_seqs], [int(w.meta["prefix_blocks"])])
            ws_bytes = pa.shared_prefix_workspace_bytes(
                w.num_seqs, w.num_heads, w.kv_heads, w.head_dim, w.block_size, w.max_seq_len,
                w.max_blocks_per_seq, *self.groups, prefix_partition_size=prefix_partition,
                partition_size=partition)
        self.ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        self.ordered = (not rank_in_kernel and not self.shared
                        and self.plan.kernel == "mfma")
        self.order = pa.longest_first(self.lens) if self.ordered else None
        # shared-prefix call: the tails' order, longest first, kept like the
        # decode's order (it changes only with the batch)
        self.sp_order = (pa.longest_tail_first(self.lens, *self.groups, w.block_size)
                         if self.shared and not index_order else None)
        self.stream = torch.cuda.current_stream()

    def step(self, i, timer=None, ev=None, decode_only=False):
        w, pa = self.w, self.pa
        kc, vc = self.pools[i % len(self.pools)]
        if w.cow_pairs.shape[0] and not decode_only:
            pa.copy_blocks(kc, vc, self.pairs)
        if w.slot_mapping.shape[0] and not self.fused and not decode_only:
            pa.kv_append(self.k_new, self.v_new, kc, vc, self.slots)
        if ev is not None:
            timer.record(ev[0], self.stream)
        kw = dict(max_seq_len=w.max_seq_len, partition_size=self.partition, out=self.out,
                  workspace=self.ws)
        if self.fused:   # one launch: the new tokens' append and the decode
            pa.decode_append(self.q, kc, vc, self.fk, self.fv, self.fslots, self.bt, self.lens,
                             w.scale, kernel=self.kernel, order=self.order, **kw)
        elif self.shared:
            pa.decode_shared_prefix(self.q, kc, vc, self.bt, self.lens, w.scale, *self.groups,
                                    prefix_partition_size=self.prefix_partition,
                                    order=self.sp_order, **kw)
        elif self.ordered:
            pa.decode_ordered(self.q, kc, vc, self.bt, self.lens, self.order, w.scale,
                              kernel=self.kernel, **kw)
        else:
            pa.decode(self.q, kc, vc, self.bt, self.lens, w.scale, kernel=self.kernel, **kw)
        if ev is not None:
            timer.record(ev[1], self.stream)

    def timed(self, steps, warmup, first=0):
        """(mean step ms, per-step decode ms array) over `steps` timed steps
        after `warmup` untimed ones, on the stream the library launches on.
        Three passes: HIP events around each decode call give the spread of
        the decode times; the step time comes from a pass with events only
        around the whole region, since a record between two launches leaves
        the GPU idle for about 2 us (the step measured 131.8 us with the
        per-call events and 127.7 us without); and the mean decode call
        (self.pass_ms) from `steps` decode calls back to back (the append
        already done, the pools still rotating), events around the pass."""
        torch = self.torch
        for i in range(warmup):
            self.step(first + i)
        torch.cuda.synchronize()
        timer = HipTimer()
        evs = [(timer.event(), timer.event()) for _ in range(steps)]
        t_start, t_end = timer.event(), timer.event()
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(first + warmup + i, timer, evs[i])
        torch.cuda.synchronize()
        dec_ms = self.np.array([timer.elapsed_ms(a, b) for a, b in evs])
        timer.record(t_start, self.stream)
        for i in range(steps):
            self.step(first + warmup + steps + i)
        timer.record(t_end, self.stream)
        torch.cuda.synchronize()
        step_ms = timer.elapsed_ms(t_start, t_end) / steps
        p_start, p_end = timer.event(), timer.event()
        torch.cuda.synchronize()
        timer.record(p_start, self.stream)
        for i in range(steps):
            self.step(first + warmup + 2 * steps + i, decode_only=True)
        timer.record(p_end, self.stream)
        torch.cuda.synchronize()
        self.pass_ms = timer.elapsed_ms(p_start, p_end) / steps
        timer.close()
        return step_ms, dec_ms

    def bytes(self):
        """(live K/V bytes the attention consumes, distinct live K/V bytes)."""
        w, W = self.w, self.W
        kv = W.decode_kv_bytes(w.seq_lens, w.kv_heads, w.head_dim, w.elem_bytes)
        uniq = W.unique_kv_bytes(w.block_tables, w.seq_lens, w.block_size, w.kv_heads,
                                 w.head_dim, w.elem_bytes)
        return kv, uniq

    def summary(self, step_ms, dec_ms):
        np = self.np
        kv, uniq = self.bytes()
        dec = self.pass_ms
        return {
            "workload": self.w.name,
            "call": ("pa_decode_shared_prefix_ordered" if self.sp_order is not None else
                     "pa_decode_shared_prefix" if self.shared else
                     ("pa_decode_append_ordered" if self.ordered else "pa_decode_append")
                     if self.fused else
                     "pa_decode_ordered" if self.ordered else "pa_decode"),
            "partition_size": self.plan.partition_size if not self.shared else self.partition,
            "num_partitions": self.plan.num_partitions,
            "decode_us": {"mean": round(dec * 1e3, 2),
                          "per_call_events": {
                              "mean": round(float(dec_ms.mean()) * 1e3, 2),
                              "median": round(float(np.median(dec_ms)) * 1e3, 2),
                              "min": round(float(dec_ms.min()) * 1e3, 2)}},
            "step_us": round(step_ms * 1e3, 2),
            "kv_GBps": round(kv / (dec * 1e-3) / 1e9, 1),
            "unique_kv_GBps": round(uniq / (dec * 1e-3) / 1e9, 1),
            "frac": round(uniq / (dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "seqs_per_s": round(self.w.num_seqs / (step_ms * 1e-3), 1),
        }


# Configurations timed after the headline in the same process: (workload,
# partition size, note).  frac = distinct live K/V bytes / decode time / 8 TB/s.
OTHER_CONFIGS = [
    ("shared_prefix", 0, "pa_decode_shared_prefix, library's split"),
    ("long_context", 512, "16 partitions of 512 tokens + reduce"),
    ("long_context", 0, "library's split"),
    ("llama70b_tp8", 0, "one GPU's share at 8-way tensor parallelism: 1 KV head, 8 query heads"),
    *[(W_name, 0, "append + decode") for W_name in
      ("sweep_b16_d64", "sweep_b16_d128", "sweep_b32_d64", "sweep_b32_d128",
       "sweep_b64_d64", "sweep_b64_d128")],
]


def other_configs(np, torch, W, pa, dev, steps=40, warmup=20):
    """Decode time and HBM fraction of every other decode configuration, then
    the paging overhead: the llama70b batch against the same batch on
    physically consecutive blocks, in alternating rounds.  The pools are the
    workloads' seeded host-filled ones, copied to the device like the
    headline's.  (Pools allocated after earlier pools were freed have
    measured up to 4 % slower whatever their contents or allocation call, so
    the measured speed of a config depends a little on what the process
    allocated before it.)"""
    res = []
    for name, part, note in OTHER_CONFIGS:
        run = DecodeRun(np, torch, W, pa, dev, name, partition=part, host_fill=True)
        s = run.summary(*run.timed(steps, warmup))
        s["note"] = note
        res.append(s)
        del run
        torch.cuda.empty_cache()
    runs = {n: DecodeRun(np, torch, W, pa, dev, n, host_fill=True)
            for n in ("llama70b", "llama70b_contiguous")}
    dec = {n: [] for n in runs}
    for r in range(6):                      # alternating rounds on one box
        for n, run in runs.items():
            _, d = run.timed(20, 3, first=r * 100)
            dec[n].extend(d.tolist())
    paged = float(np.mean(dec["llama70b"]))
    contig = float(np.mean(dec["llama70b_contiguous"]))
    overhead = {
        "random_placement_us": round(paged * 1e3, 2),
        "sequential_placement_us": round(contig * 1e3, 2),
        "overhead_pct": round(100.0 * (paged / contig - 1.0), 2),
        "method": "pa_decode_ordered on the llama70b batch with random block placement vs "
                  "the same batch on consecutive blocks, 6 alternating rounds of 20 steps",
    }
    return res, overhead


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (--gpus {args.gpus} requested); "
              "the decode path shards by sequence or KV head with no exchange, but no "
              "multi-GPU run is provided.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_163_amd import build as B
    from paged_kv_cache_163_amd import workloads as W
    if not os.path.exists(B.LIB):
        B.build()
    from paged_kv_cache_163_amd import pa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload in W.PREFILL_WORKLOADS:
        return prefill_main(args, np, torch, W, pa, dev)
    if args.workload == "swap_llama70b":
        return swap_main(args, np, torch, W, pa, dev)
    if args.workload == "layered_llama70b":
        return layered_main(args, np, torch, W, pa, dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    run = DecodeRun(np, torch, W, pa, dev, args.workload, rotate=args.rotate,
                    partition=args.partition, kernel=args.kernel, fused=args.fused_append,
                    rank_in_kernel=args.rank_in_kernel, plain_decode=args.plain_decode,
                    prefix_partition=args.prefix_partition, host_fill=True,
                    index_order=args.index_order)
    w, plan = run.w, run.plan
    step_ms, dec_ms = run.timed(args.steps, args.warmup)

    kv_bytes, unique_bytes = run.bytes()
    total_alg = (kv_bytes + 2 * w.q.nbytes + 4 * int(sum(-(-int(n) // w.block_size)
                                                        for n in w.seq_lens)) + 4 * w.num_seqs)
    value = kv_bytes / (step_ms * 1e-3) / 1e9
    fused, shared, ordered = run.fused, run.shared, run.ordered
    nparts = plan.num_partitions
    kernel_name = f"decode_{plan.kernel}_kernel" + (" (fused append)" if fused else "")
    split_reduce = nparts > 1
    if shared:
        kernel_name = "shared_prefix_kernel (prefix + tails) + prefix_merge_kernel"
        split_reduce = False
    dec_avg = run.pass_ms
    # distinct live K/V bytes over the decode call: when tables share blocks, what
    # one pass over the pool must read (equal to kv_bytes otherwise)
    achieved = unique_bytes / (dec_avg * 1e-3) / 1e9
    # the stored counter record is for the plain decode kernel at the default plan
    plain = args.partition == 0 and args.kernel == "auto" and not fused
    traffic = None
    if plain and shared and args.prefix_partition == 0:
        traffic = traffic_entry(w.name, "shared_prefix_kernel")
    elif plain and not shared:
        traffic = traffic_entry(w.name)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs,
            "num_heads": w.num_heads,
            "kv_heads": w.kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "num_blocks": w.num_blocks,
            "mean_seq_len": round(float(w.seq_lens.mean()), 2),
            "max_seq_len": w.max_seq_len,
            "appended_tokens": int(w.slot_mapping.shape[0]),
            "append": "fused into the decode launch" if fused else "pa_kv_append launch",
            "order": ("longest-first, kept across steps (pa_decode_ordered)" if ordered
                      else ("tails longest first (pa_decode_shared_prefix_ordered)"
                            if run.sp_order is not None else "index order (shared-prefix decode)")
                      if shared
                      else "ranked inside the kernel"),
            "shared_prefix": ({"call": ("pa_decode_shared_prefix" if run.sp_order is None else
                                        "pa_decode_shared_prefix_ordered"),
                               "tail_order": ("index" if run.sp_order is None else
                                              "longest tail first, kept across steps"),
                               "groups": run.groups[0],
                               "prefix_blocks": run.groups[1],
                               "prefix_partition": args.prefix_partition or "library's choice"}
                              if shared else None),
            "cow_pairs": int(w.cow_pairs.shape[0]),
            "kernel": plan.kernel,
            "partition_size": plan.partition_size,
            "num_partitions": nparts,
            "pool_rotation": len(run.pools),
            "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(w.num_seqs / (step_ms * 1e-3), 1),
        "decode_ms": {"mean": round(dec_avg, 5),
                      "per_call_events": {"mean": round(float(dec_ms.mean()), 5),
                                          "median": round(float(np.median(dec_ms)), 5),
                                          "min": round(float(dec_ms.min()), 5)}},
        "kv_bytes_per_step": kv_bytes,
        "unique_kv_bytes_per_step": unique_bytes,
        "total_algorithmic_bytes_per_decode": total_alg,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": kernel_name + (" + decode_reduce_kernel" if split_reduce else ""),
            "bytes_per_launch": unique_bytes,
            "avg_launch_ms": round(dec_avg, 5),
        },
        "cpu_baseline": None,
    }
    if args.power_seconds > 0:
        line["power"] = sample_power(torch, run.step, args.power_seconds)
    if not args.no_other_configs and args.workload == "llama70b":
        del run
        torch.cuda.empty_cache()
        others, paging = other_configs(np, torch, W, pa, dev)
        line["other_configs"] = others
        line["paging_overhead"] = paging
        # the two prefill batches, steady state (each warms up for 300 ms first)
        pf = []
        for name in ("prefill_llama70b", "prefill_chunked"):
            w_p, ms_p, _, _ = prefill_timed(np, torch, W, pa, dev, name, 100, 10, 300.0, 4)
            pf.append(prefill_line(W, w_p, ms_p))
            torch.cuda.empty_cache()
        line["prefill"] = pf
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
