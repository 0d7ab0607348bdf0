"""Benchmark of the grouped row-scaled NVFP4 amax + cast on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Timing: untimed steps for --settle-ms (the clocks of a fresh GPU ramp up
under load), then --warmup untimed steps, then exactly --steps timed steps
between two device synchronisations; per-kernel times come from HIP events
recorded on the launch stream.

A step is one pass of the whole path over the workload: the grouped amax
(rowwise + per-expert columnwise) then the grouped cast (rowwise +
transposed), through the C ABI, with the input resident in HBM.  The default
workload is the DeepSeek-V3-style one-GPU expert share (32 experts, K=7168,
sum_M=65536, Zipf routing, both directions).  Prints one JSON line.

value = algorithmic bytes per step / time per step, where the algorithmic
bytes count what the method must move: two reads of x (the column amax needs
every row of an expert before any of its blocks can be cast), the amax
vectors written once and read once, and both outputs written once.

Beside the headline the line carries:
- ``configs``: the other workloads -- tiny (4 experts, one launch), outliers
  (rowwise only, one fused pass), down_proj (64 experts, K=2048) -- each
  timed with the same protocol, and graph_replay: one hipGraph capture of the
  graph-safe step on the expert-share shapes replayed with 100 seeded
  routings (timed back to back, then every routing checked byte for byte
  against the host-split path on the device);
- ``flushed_step``: the same steps with a 512 MB read before each (outside
  the events), so that the 256 MB memory-side cache holds nothing of the
  step's data and no dirty lines of the previous step;
- ``hbm_ceiling``: what this memory system moves with kernels written here
  (read, fill, copy with the best grid of a sweep, the cast's read/write
  ratio in a contiguous layout, and the cast's own memory pattern with the
  arithmetic removed) and torch's device copy;
- ``next_rows``: the grouped MXFP4 cast of the same input, the rowwise /
  columnwise NVFP4 dequant of the step's outputs, the four-over-six cast of
  the same input (vector-ALU-bound), and the row-scaled grouped
  GEMM (forward and weight gradient, MFMA-bound, TFLOP/s against the fp16
  MFMA peak) with torch.matmul (hipBLASLt) fp16 on the same shapes beside it;
- ``cpu_baseline``: the CPU oracle over the whole workload on the host's
  threads (at most 16), timed before the process touches the GPU; each
  entry of ``configs`` carries the same figure for its own workload
  (median of 5 runs for the two small ones).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
EVENT_STRIDE = 10  # timed steps per step with per-launch events
METRIC = "grouped NVFP4 amax+cast HBM GB/s (bytes in+out) and % of MI355X peak BW"
# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, per workload
TRAFFIC_FILES = {"deepseek_share": "profiles/group_cast_kernel-deepseek_share_e32_k7168_m65536.md",
                 "down_proj": "profiles/group_cast_kernel-down_proj_e64_k2048_m131072.md",
                 "tiny": "profiles/group_quantize_small_kernel-tiny_e4_k256_m512.md",
                 "outliers": "profiles/group_quantize_rowwise_kernel-outliers_e8_k2048_m8192_rowwise.md"}


class TimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence.

    A default HIP event performs a system-scope fence when it is recorded
    (a cache write-back and invalidate, which also slows the kernel that
    follows); timing events need none of that: the host reads results only
    after a device synchronisation.  Events are recorded on the stream the
    library launches on (torch's current stream) through the HIP runtime
    that torch has loaded."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.hip = ctypes.CDLL(path)
        self.torch = torch
        self.pool = []

    def new(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.pool.append(ev)
        return ev

    def record(self, ev):
        rc = self.hip.hipEventRecord(ev, self._stream())
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def _stream(self):
        raw = getattr(self.torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:  # the current stream's handle, without building a Stream object
            return ctypes.c_void_p(raw(self.torch.cuda.current_device()))
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for ev in self.pool:
            self.hip.hipEventDestroy(ev)
        self.pool = []


def algorithmic_bytes(sum_m: int, k: int, E: int, rowwise: bool, columnwise: bool) -> dict:
    N = sum_m * k
    if rowwise and not columnwise:
        # one fused pass: read x once, write the row amax and the rowwise output
        fused = 2 * N + 4 * sum_m + N // 2 + N // 16
        return {"fused_kernel": fused, "step": fused}
    amax_out = (4 * sum_m if rowwise else 0) + (4 * E * k if columnwise else 0)
    outs = (N // 2 + N // 16) * (int(rowwise) + int(columnwise))
    amax_k = 2 * N + amax_out                     # read x, write amax
    cast_k = 2 * N + amax_out + outs              # read x and amax, write data + scales
    return {"amax_kernel": amax_k, "cast_kernel": cast_k, "step": amax_k + cast_k}


def host_cpu() -> dict:
    """What the host offers the CPU baseline: CPU model, online CPUs, the CPUs
    this process may run on, and the worker threads the oracle uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": affinity}


def cpu_baseline(w, one_thread_rows: int = 16384, threads: int | None = None, reps: int = 1) -> dict:
    """The oracle, as it stands, on the whole workload: independent oracle
    calls (the rowwise direction on row ranges, the columnwise direction on
    column ranges of each expert; together exactly the bytes of one call) on
    a pool of host threads, at most one per CPU of the process's share and at
    most 16 (a one-GPU share of the GPU host).  Also one call on one thread
    over the first whole experts (in expert order) that fit in
    ``one_thread_rows`` rows.  Each timing is the median of ``reps`` runs.
    Runs before the process touches the GPU."""
    from oracle import oracle as O
    from oracle import parallel as OP
    n = threads or OP.default_threads()

    def med(fn):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    dtn = med(lambda: OP.group_quantize(w.x, w.splits, w.rowwise, w.columnwise, threads=n))
    b_all = algorithmic_bytes(w.sum_m, w.k, w.num_experts, w.rowwise, w.columnwise)["step"]
    offs = np.concatenate([[0], np.cumsum(w.splits)])
    chosen, rows = [], 0
    for e, m in enumerate(w.splits):
        if m and rows + int(m) <= one_thread_rows:
            chosen.append(e)
            rows += int(m)
    xs = np.concatenate([w.x[offs[e]:offs[e + 1]] for e in chosen])
    sp = [int(w.splits[e]) for e in chosen]
    dt1 = med(lambda: O.group_quantize(xs, sp, w.rowwise, w.columnwise))
    b1 = algorithmic_bytes(rows, w.k, len(sp), w.rowwise, w.columnwise)["step"]
    ntasks = len(OP.tasks(w.splits, w.k, w.rowwise, w.columnwise))
    res = {"value": round(b_all / dtn / 1e9, 5), "unit": "GB/s", "cores": n, "kind": "oracle",
           "sample": f"the whole workload ({w.sum_m} rows x K={w.k}, {directions(w)}): {ntasks} row-range / "
                     f"column-range calls of the C oracle on {n} threads, {dtn:.3f} s"
                     + (f" (median of {reps} runs)" if reps > 1 else ""),
           "seconds": round(dtn, 3), "threads": n,
           "value_one_thread": round(b1 / dt1 / 1e9, 5),
           "one_thread_sample": f"one call on one thread: {len(sp)} whole experts, {rows} rows, {dt1:.3f} s"}
    res.update(host_cpu())
    return res


WORKLOADS = ["deepseek_share", "down_proj", "outliers", "tiny"]
# the other configurations reported beside the headline, with their timed
# steps and the runs of the CPU oracle timed for each (median)
SIDE_CONFIGS = {"tiny": 1000, "outliers": 1000, "down_proj": 200}
SIDE_CPU_REPS = {"tiny": 5, "outliers": 5, "down_proj": 1}


def measure_step(B, torch, tev, w, x, out, steps: int, warmup: int, settle_ms: float) -> dict:
    """Time `steps` back-to-back steps of the whole path on workload `w` (x and
    the outputs already on the device): wall clock between two device
    synchronisations, plus per-launch times from HIP events on the stream
    around the launches of every EVENT_STRIDE-th of those steps."""
    splits = [int(v) for v in w.splits]
    k = w.k
    fused = w.rowwise and not w.columnwise
    # small inputs with a columnwise output: the library's one-launch path
    small = w.columnwise and max(splits) * k <= B.SMALL_MAX_EXPERT_ELEMS and k <= B.SMALL_MAX_K

    def step(ev=None):
        if ev is not None:
            tev.record(ev[0])
        if fused or small:
            # rowwise only: one pass (row amax and cast together); small
            # inputs: one launch, eight work-groups per expert
            B.nvfp4_group_quantize(x, splits, **out)
            if ev is not None:
                tev.record(ev[1])
                tev.record(ev[2])
            return
        B.nvfp4_group_amax(x, splits, out["row_amax"], out["col_amax"])
        if ev is not None:
            tev.record(ev[1])
        B.nvfp4_group_cast(x, splits, **out)
        if ev is not None:
            tev.record(ev[2])

    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # HIP events around the launches of every EVENT_STRIDE-th timed step give
    # the per-kernel times: an event record costs a few microseconds of
    # stream time, which around every step would add ~2% to the expert-share
    # step and half again to the small ones
    events = {i: [tev.new() for _ in range(3)] for i in range(0, steps, EVENT_STRIDE)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    first_ms = float(np.mean([tev.elapsed_ms(e[0], e[1]) for e in events.values()]))
    second_ms = float(np.mean([tev.elapsed_ms(e[1], e[2]) for e in events.values()]))
    nbytes = algorithmic_bytes(w.sum_m, k, w.num_experts, w.rowwise, w.columnwise)
    ms_per_step = wall * 1e3 / steps
    if fused or small:
        dom_name = "group_quantize_rowwise_kernel" if fused else "group_quantize_small_kernel"
        dom_ms, dom_bytes = first_ms, nbytes["fused_kernel"] if fused else nbytes["step"]
        kernels = {dom_name: {"avg_us": round(dom_ms * 1e3, 2), "GBps": round(dom_bytes / dom_ms / 1e6, 2)}}
        entry = ("nvfp4_group_quantize (host splits, fused rowwise pass)" if fused
                 else "nvfp4_group_quantize (host splits, one launch for a small input)")
    else:
        dom_name, dom_ms, dom_bytes = "group_cast_kernel", second_ms, nbytes["cast_kernel"]
        amax_name = "group_amax_rows_kernel" if k <= 2048 else "group_amax_kernel"
        kernels = {f"amax (init + {amax_name})": {"avg_us": round(first_ms * 1e3, 2),
                                                  "GBps": round(nbytes["amax_kernel"] / first_ms / 1e6, 2)},
                   "group_cast_kernel": {"avg_us": round(second_ms * 1e3, 2),
                                         "GBps": round(nbytes["cast_kernel"] / second_ms / 1e6, 2)}}
        entry = "nvfp4_group_amax + nvfp4_group_cast (host splits)"
    return {"steps": steps, "ms_per_step": ms_per_step, "first_ms": first_ms, "second_ms": second_ms,
            "nbytes": nbytes, "dom_name": dom_name, "dom_ms": dom_ms, "dom_bytes": dom_bytes,
            "kernels": kernels, "entry": entry, "step": step}


def directions(w) -> str:
    return "+".join(d for d, on in (("rowwise", w.rowwise), ("columnwise", w.columnwise)) if on)


def roofline(profiling, workload: str, kernel: str, nbytes: int, ms: float) -> dict:
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic_file = TRAFFIC_FILES.get(workload)
    traffic = profiling.load_traffic(os.path.join(ROOT, traffic_file), kernel) if traffic_file else None
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic["bytes"] if traffic else None,
            "traffic_source": traffic_file if traffic else None, "avg_us": round(ms * 1e3, 2),
            "algorithmic_bytes_per_launch": nbytes}


def side_config(B, torch, tev, profiling, dev, w, name: str, steps: int, cpu=None) -> dict:
    """One of the other configurations: the same step protocol (shorter), its
    rate against the HBM peak, the kernels' event times, (where a profile
    exists) the dominant kernel's measured traffic, and the CPU oracle's rate
    on the same workload (timed before any GPU use)."""
    print(f"[bench] config {name}", file=sys.stderr, flush=True)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    out = B.alloc_outputs(w.sum_m, w.k, w.num_experts, w.rowwise, w.columnwise, device=dev)
    r = measure_step(B, torch, tev, w, x, out, steps, max(20, steps // 10), 30.0)
    gbs = r["nbytes"]["step"] / (r["ms_per_step"] * 1e-3) / 1e9
    res = {"workload": w.name, "directions": directions(w), "entry": r["entry"], "steps": steps,
           "ms_per_step": round(r["ms_per_step"], 5), "GBps": round(gbs, 2),
           "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_step": r["nbytes"]["step"],
           "gpu_ms_per_step": round(r["first_ms"] + r["second_ms"], 5), "kernels": r["kernels"],
           "roofline": roofline(profiling, name, r["dom_name"], r["dom_bytes"], r["dom_ms"])}
    if cpu is not None:
        res["cpu_baseline"] = cpu
    del x, out
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed steps for this long before the warmup steps: the GPU's clocks ramp up over "
                         "the first tens of milliseconds of load on a fresh box (0: skip)")
    ap.add_argument("--workload", default="deepseek_share", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations")
    ap.add_argument("--graph-replays", type=int, default=100)
    ap.add_argument("--next-rows", type=int, default=20,
                    help="launches timed for each of the MXFP4 cast and the two dequants (0: skip)")
    ap.add_argument("--next-only", default=None, choices=("mxfp4", "dequant", "four_over_six", "gemm"),
                    help="run only this group of next rows (for profiling one kernel)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="also time the steps with a read of this many MB before each (outside the timed "
                         "events), so that no input or output is left in the 256 MB memory-side cache (0: skip)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the memory-ceiling kernels")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (3 times, untimed) so that a "
                         "rocprofv3 --pmc run can scale FETCH_SIZE / WRITE_SIZE by a copy of known size")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    from nvfp4_block_scaled_group_amd import synth

    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    w = synth.CONFIGS[args.workload]()
    cpu = None
    side = {} if args.no_configs else {name: synth.CONFIGS[name]() for name in SIDE_CONFIGS if name != args.workload}
    side_cpu = {}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (before any GPU use)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)
        for name, sw in side.items():
            side_cpu[name] = cpu_baseline(sw, reps=SIDE_CPU_REPS[name])

    import torch
    from nvfp4_block_scaled_group_amd import binding as B
    from nvfp4_block_scaled_group_amd import profiling

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    splits = [int(v) for v in w.splits]
    E, k, m = w.num_experts, w.k, w.sum_m
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    out = B.alloc_outputs(m, k, E, w.rowwise, w.columnwise, device=dev)
    tev = TimingEvents(torch)

    print(f"[bench] settle {args.settle_ms:.0f} ms, warmup {args.warmup}, timing {args.steps} steps",
          file=sys.stderr, flush=True)
    r = measure_step(B, torch, tev, w, x, out, args.steps, args.warmup, args.settle_ms)
    ms_per_step, nbytes, step = r["ms_per_step"], r["nbytes"], r["step"]
    value = nbytes["step"] / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "num_experts": E, "k": k, "sum_m": m, "directions": directions(w),
                   "entry": r["entry"], "algorithmic_bytes_per_step": nbytes["step"],
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": roofline(profiling, args.workload, r["dom_name"], r["dom_bytes"], r["dom_ms"]),
        "kernels": r["kernels"],
    }

    if args.flush_mb > 0:
        # the same steps with a read of flush_mb MB (twice the 256 MB MALL by
        # default) before each, outside the events: nothing of x or of the
        # previous step's outputs is left in the memory-side cache.  A read
        # (a max reduction) rather than a fill: a fill would leave dirty lines
        # whose write-back the next step would pay for.
        flush = torch.ones(args.flush_mb << 17, dtype=torch.int64, device=dev)
        flush.max()
        torch.cuda.synchronize()
        fev = [[tev.new() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            flush.max()
            step(fev[i])
        torch.cuda.synchronize()
        f_all = [tev.elapsed_ms(e[0], e[2]) for e in fev]
        f_ms = float(np.mean(f_all))
        f1 = float(np.mean([tev.elapsed_ms(e[0], e[1]) for e in fev]))
        result["flushed_step"] = {"flush_mb": args.flush_mb, "steps": args.steps,
                                  "ms_per_step": round(f_ms, 4), "median_ms": round(float(np.median(f_all)), 4),
                                  "min_ms": round(float(np.min(f_all)), 4),
                                  "GBps": round(nbytes["step"] / (f_ms * 1e-3) / 1e9, 2),
                                  "first_launch_us": round(f1 * 1e3, 2),
                                  "second_launch_us": round((f_ms - f1) * 1e3, 2),
                                  "unflushed_event_ms_per_step": round(r["first_ms"] + r["second_ms"], 4)}
        del flush

    if not args.no_ceiling:
        result["hbm_ceiling"] = hbm_ceiling(torch, tev, dev, w, x, out)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if w.rowwise and w.columnwise and args.next_rows > 0:
        result["next_rows"] = next_rows(B, torch, tev, x, splits, out, E, k, m, args.next_rows, args.next_only)
    del x, out
    torch.cuda.empty_cache()

    if not args.no_configs:
        configs = {}
        for name, sw in side.items():
            configs[name] = side_config(B, torch, tev, profiling, dev, sw, name, SIDE_CONFIGS[name],
                                        side_cpu.get(name))
        if args.graph_replays > 0:
            configs["graph_replay"] = graph_replay(B, synth, torch, tev, dev, args.graph_replays)
        result["configs"] = configs

    if cpu is not None:
        result["cpu_baseline"] = cpu
    tev.close()
    print(json.dumps(result), flush=True)


class Probe:
    """The memory-ceiling kernels of probe/libhbmprobe.so, on torch's current stream."""

    def __init__(self, tev):
        path = os.path.join(ROOT, "nvfp4_block_scaled_group_amd", "probe", "libhbmprobe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m nvfp4_block_scaled_group_amd.build`")
        self.L = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        self.L.hbm_probe_read.argtypes = [P, I64, P, I, P]
        self.L.hbm_probe_fill.argtypes = [P, I64, I, P]
        self.L.hbm_probe_copy.argtypes = [P, P, I64, I, P]
        self.L.hbm_probe_mix.argtypes = [P, P, I64, I, P]
        self.L.hbm_probe_cast_pattern.argtypes = [P, I64, I64, ctypes.c_int32, P, P, P, P, P, P]
        self.tev = tev

    def call(self, fn, *args):
        rc = getattr(self.L, fn)(*args, self.tev._stream())
        if rc != 0:
            raise RuntimeError(f"{fn} failed ({rc})")


def hbm_ceiling(torch, tev, dev, w, x, out, reps: int = 10) -> dict:
    """Context for roofline.frac, measured in the same process with kernels
    written here (probe/hbm_probe.hip): a 1 GiB read, fill and copy (the best
    grid of a sweep), the cast's read/write ratio in its simplest layout
    (64 KB read and 36 KB written contiguously per work-group), and the
    cast's own loads and stores with no arithmetic, on this workload's
    buffers; torch's device copy beside them."""
    print("[bench] memory ceiling", file=sys.stderr, flush=True)
    pr = Probe(tev)
    G = 1 << 30
    src = torch.empty(G, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def timed(fn):
        # the kernel alone for ~50 ms first: clocks ramp up under sustained
        # load (the first launches after host work run up to 20% slower)
        t_end = time.perf_counter() + 0.05
        while time.perf_counter() < t_end:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
        evs = [(tev.new(), tev.new()) for _ in range(reps)]
        for e0, e1 in evs:
            tev.record(e0)
            fn()
            tev.record(e1)
        torch.cuda.synchronize()
        return float(np.mean([tev.elapsed_ms(a, b) for a, b in evs]))

    def rate(name, ms, nbytes, **extra):
        gbs = nbytes / (ms * 1e-3) / 1e9
        d = {"kind": name, "avg_us": round(ms * 1e3, 2), "bytes": nbytes, "GBps": round(gbs, 2),
             "frac": round(gbs / HBM_PEAK_GBS, 4)}
        d.update(extra)
        return d

    def best(fn_of_grid, grids=(512, 1024, 2048, 4096, 8192)):
        times = {g: timed(lambda g=g: fn_of_grid(g)) for g in grids}
        g = min(times, key=times.get)
        return times[g], g

    res = {}
    ms, g = best(lambda g: pr.call("hbm_probe_read", p(src), G, p(sink), g))
    res["read"] = rate("1 GiB read, non-temporal 16-byte loads", ms, G, grid=g)
    ms, g = best(lambda g: pr.call("hbm_probe_fill", p(dst), G, g))
    res["fill"] = rate("1 GiB written, streaming 16-byte stores", ms, G, grid=g)
    ms, g = best(lambda g: pr.call("hbm_probe_copy", p(src), p(dst), G, g))
    res["copy"] = rate("1 GiB read + 1 GiB written, non-temporal loads and streaming stores", ms, 2 * G, grid=g)
    ms = timed(lambda: pr.call("hbm_probe_mix", p(src), p(dst), G, 9))
    res["cast_ratio_mix"] = rate("1 GiB read + 576 MiB written (64 KB read and 36 KB written contiguously per "
                                 "work-group, the cast's ratio)", ms, G + G // 16 * 9)
    ms = timed(lambda: dst.copy_(src))
    res["torch_copy"] = rate("torch device copy_, 1 GiB read + 1 GiB written", ms, 2 * G)
    del src, dst
    torch.cuda.empty_cache()
    if w.rowwise and w.columnwise and w.k % 256 == 0 and w.num_experts <= 512:
        sp = (ctypes.c_int64 * w.num_experts)(*[int(v) for v in w.splits])
        N = w.sum_m * w.k
        ms = timed(lambda: pr.call("hbm_probe_cast_pattern", p(x), w.sum_m, w.k, w.num_experts, sp,
                                   p(out["row_data"]), p(out["row_scale"]), p(out["col_data"]),
                                   p(out["col_scale"])))
        res["cast_pattern_no_arithmetic"] = rate(
            "the cast kernel's loads and stores on this workload's buffers, no arithmetic", ms,
            2 * N + 2 * (N // 2 + N // 16))
    return res


def next_rows(B, torch, tev, x, splits, out, E: int, k: int, m: int, reps: int, only=None) -> dict:
    """MXFP4 cast of the step's input and NVFP4 dequant of its outputs."""
    print("[bench] MXFP4 cast and dequant", file=sys.stderr, flush=True)
    N = m * k

    def timed(fn):
        # the kernel alone for ~50 ms first: clocks ramp up under sustained
        # load (the first launches after host work run up to 20% slower)
        t_end = time.perf_counter() + 0.05
        while time.perf_counter() < t_end:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
        evs = [(tev.new(), tev.new()) for _ in range(reps)]
        for e0, e1 in evs:
            tev.record(e0)
            fn()
            tev.record(e1)
        torch.cuda.synchronize()
        return float(np.mean([tev.elapsed_ms(a, b) for a, b in evs]))

    def entry(kernel, ms, nbytes):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"kernel": kernel, "avg_us": round(ms * 1e3, 2), "algorithmic_bytes_per_launch": nbytes,
                "GBps": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4)}

    res = {}
    if only in (None, "mxfp4"):
        mx = B.alloc_mx_outputs(m, k, device=x.device)
        ms = timed(lambda: B.mxfp4_group_cast(x, splits, **mx))
        res["mxfp4_group_cast"] = entry("mxfp4_group_cast_kernel", ms, 2 * N + 2 * (N // 2 + N // 32))
        del mx
    if only in (None, "dequant"):
        deq = torch.empty(N, dtype=torch.float32, device=x.device)
        ms = timed(lambda: B.nvfp4_group_dequant_rowwise(out["row_data"], out["row_scale"], out["row_amax"],
                                                          deq.view(m, k)))
        res["nvfp4_group_dequant_rowwise"] = entry("dequant_kernel", ms, N // 2 + N // 16 + 4 * m + 4 * N)
        ms = timed(lambda: B.nvfp4_group_dequant_columnwise(out["col_data"], out["col_scale"], out["col_amax"],
                                                             splits, k, deq))
        res["nvfp4_group_dequant_columnwise"] = entry("dequant_kernel", ms, N // 2 + N // 16 + 4 * E * k + 4 * N)
        del deq
    if only in (None, "four_over_six"):
        res.update(four_over_six_rows(B, torch, timed, entry, x, splits, out, E, k, m))
    if only in (None, "gemm"):
        res.update(gemm_rows(B, torch, timed, out, splits, E, k, m))
    return res


# fp32 operations the four-over-six method performs per element, direction
# and candidate: x*m, value(code)*value(S), *s, the difference, its square
# (or absolute value) and the running sum
FOUR_OVER_SIX_OPS = 6
# non-packed fp32 VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_LANE_OPS_PEAK_T = 256 * 4 * 16 * 2.4e9 / 1e12


def four_over_six_rows(B, torch, timed, entry, x, splits, out, E: int, k: int, m: int) -> dict:
    """The four-over-six cast of the step's input (both directions, default
    bound 256, squared and absolute error), consuming the step's amax.  The
    kernel is bound by the vector ALUs: beside the HBM figures it reports the
    method's fp32 operations per second against the non-packed VALU rate."""
    print("[bench] four-over-six cast", file=sys.stderr, flush=True)
    N = m * k
    res = {}
    o = B.alloc_outputs(m, k, E, device=x.device)
    o["row_amax"], o["col_amax"] = out["row_amax"], out["col_amax"]
    for mode, tag in ((B.ERR_MSE, "mse"), (B.ERR_MAE, "mae")):
        ms = timed(lambda: B.nvfp4_group_cast_4over6(x, splits, **o, scale_bound=B.DEFAULT_4O6_BOUND,
                                                      err_mode=mode))
        r = entry("group_cast_4o6_kernel", ms, 2 * N + 2 * (N // 2 + N // 16) + 4 * m + 4 * E * k)
        ops = 2 * 2 * FOUR_OVER_SIX_OPS * N
        r["alu"] = {"bound": "alu", "method_fp32_ops_per_launch": ops,
                    "achieved_Tops": round(ops / (ms * 1e-3) / 1e12, 2), "peak_Tops": VALU_LANE_OPS_PEAK_T,
                    "frac": round(ops / (ms * 1e-3) / 1e12 / VALU_LANE_OPS_PEAK_T, 4)}
        res[f"nvfp4_group_cast_4over6_{tag}"] = r
    del o
    return res


GEMM_N = 2048          # a DeepSeek-V3 expert's gate projection: hidden 7168 -> intermediate 2048
MFMA_F16_PEAK_TFLOPS = 2500.0


def gemm_rows(B, torch, timed, out, splits, E: int, k: int, m: int) -> dict:
    """Row-scaled grouped GEMM on the step's outputs: the forward product of
    the rowwise cast (A) with per-expert NVFP4 weights [E, GEMM_N, k], and the
    weight gradient of the columnwise cast (B) with a columnwise dY operand.
    Weight and dY operands are seeded random FP4 codes, finite E4M3 scales
    and positive amax (the kernels' time does not depend on the values)."""
    print("[bench] grouped GEMM", file=sys.stderr, flush=True)
    if k % 128:
        return {}
    dev = out["row_data"].device
    n = GEMM_N
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    codes = lambda *shape: torch.randint(0, 256, shape, dtype=torch.uint8, device=dev, generator=g)
    scales = lambda *shape: torch.randint(0x20, 0x50, shape, dtype=torch.uint8, device=dev, generator=g)
    amax = lambda n_: torch.rand(n_, device=dev, generator=g) + 0.5
    flops = 2.0 * m * n * k

    def entry(kernel, ms):
        tf = flops / (ms * 1e-3) / 1e12
        return {"kernel": kernel, "avg_us": round(ms * 1e3, 2), "flops_per_launch": flops,
                "shape": {"sum_m": m, "n": n, "k": k, "num_experts": E},
                "TFLOPs": round(tf, 1), "bound": "mfma", "peak_TFLOPs": MFMA_F16_PEAK_TFLOPS,
                "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}

    res = {}
    w = (codes(E, n, k // 2), scales(E, n, k // 16), amax(E * n))
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    ms = timed(lambda: B.nvfp4_group_gemm(out["row_data"], out["row_scale"], out["row_amax"], *w, splits, y))
    res["nvfp4_group_gemm"] = entry("gemm_fwd_kernel", ms)
    del w, y
    dy = (codes(m * n // 2), scales(m * n // 16), amax(E * n))
    dw = torch.empty((E, n, k), dtype=torch.float32, device=dev)
    ms = timed(lambda: B.nvfp4_group_gemm_wgrad(*dy, out["col_data"], out["col_scale"], out["col_amax"], splits,
                                                n, k, dw))
    res["nvfp4_group_gemm_wgrad"] = entry("gemm_wgrad_kernel", ms)
    del dy, dw
    res["library_fp16"] = library_gemm_rows(torch, timed, splits, n, k, m, dev)
    return res


def library_gemm_rows(torch, timed, splits, n: int, k: int, m: int, dev) -> dict:
    """Context for the grouped GEMM's rate: torch.matmul (hipBLASLt) in fp16 on
    operands of the same shapes, already decoded (no FP4 decode, fp16 output,
    half the output bytes of the fp32 kernels).  Per expert as a loop of
    GEMMs (what a grouped product costs through the library), and the forward
    as one dense GEMM over all rows with one weight (an upper bound: no
    grouping).  Not part of the path."""
    print("[bench] library fp16 GEMMs (context)", file=sys.stderr, flush=True)
    flops = 2.0 * m * n * k
    offs = np.concatenate([[0], np.cumsum(splits)]).tolist()
    live = [(e, offs[e], offs[e + 1]) for e in range(len(splits)) if splits[e]]
    h = torch.float16
    a = torch.randn(m, k, dtype=h, device=dev)
    wts = torch.randn(len(splits), n, k, dtype=h, device=dev)
    dyt = torch.randn(n, m, dtype=h, device=dev)

    def fwd_loop():
        for e, r0, r1 in live:
            torch.matmul(a[r0:r1], wts[e].t())

    def wgrad_loop():
        for _, r0, r1 in live:
            torch.matmul(dyt[:, r0:r1], a[r0:r1])

    def rate(ms):
        return {"avg_us": round(ms * 1e3, 2), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1)}

    res = {"grouped_fwd_loop": rate(timed(fwd_loop))}
    if hasattr(torch, "_grouped_mm"):  # torch's grouped GEMM (offsets = inclusive row ends)
        ends = torch.tensor(offs[1:], dtype=torch.int32, device=dev)
        res["grouped_fwd_torch_grouped_mm"] = rate(timed(lambda: torch._grouped_mm(a, wts.transpose(-2, -1),
                                                                                   offs=ends)))
    res["dense_fwd_one_gemm"] = rate(timed(lambda: torch.matmul(a, wts[0].t())))
    res["grouped_wgrad_loop"] = rate(timed(wgrad_loop))
    del a, wts, dyt
    return res


def graph_replay(B, synth, torch, tev, dev, replays: int) -> dict:
    """Graph-safe path on the expert-share shapes with gradient-like values:
    one hipGraph capture of amax + cast, replayed with new seeded routing
    written to the device offsets before each replay (outside the timed
    launch), back to back.  Then every routing is replayed again and
    checked: the graph's outputs and a second output set are filled with
    different sentinel bytes first; after the replay the host-split path
    writes the second set for the same routing and the two are compared on
    the device, so a byte left unwritten by either differs."""
    print("[bench] graph replay workload", file=sys.stderr, flush=True)
    w = synth.graph_replay()
    E, k, m = w.num_experts, w.k, w.sum_m
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    out = B.alloc_outputs(m, k, E, True, True, device=dev)
    host = B.alloc_outputs(m, k, E, True, True, device=dev)
    route_splits = [[int(v) for v in synth.replay_splits(i)] for i in range(replays)]
    routes = [torch.tensor(B.offsets_from_splits(sp), dtype=torch.int32).pin_memory() for sp in route_splits]
    d_offs = torch.empty(E, dtype=torch.int32, device=dev)
    d_status = torch.zeros(1, dtype=torch.int32, device=dev)
    d_offs.copy_(routes[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.nvfp4_group_quantize_graphsafe(x, E, d_offs, d_status, **out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.nvfp4_group_quantize_graphsafe(x, E, d_offs, d_status, **out)
    torch.cuda.synchronize()
    keys = [key for key, t in out.items() if t is not None]
    # timing: replays back to back, new routing copied in before each
    times = []
    for i in range(replays):
        d_offs.copy_(routes[i], non_blocking=True)
        e0, e1 = tev.new(), tev.new()
        tev.record(e0)
        g.replay()
        tev.record(e1)
        times.append((e0, e1))
    torch.cuda.synchronize()
    # verification: the same routings again, each replay's outputs compared
    # with the host-split path after sentinel fills
    identical = 0
    for i in range(replays):
        d_offs.copy_(routes[i], non_blocking=True)
        for key in keys:
            out[key].view(torch.uint8).fill_(0xA5)
            host[key].view(torch.uint8).fill_(0x5A)
        g.replay()
        B.nvfp4_group_amax(x, route_splits[i], host["row_amax"], host["col_amax"])
        B.nvfp4_group_cast(x, route_splits[i], **host)
        identical += int(all(torch.equal(out[key], host[key]) for key in keys))
    torch.cuda.synchronize()
    ms = float(np.mean([tev.elapsed_ms(a, b) for a, b in times]))
    nbytes = algorithmic_bytes(m, k, E, True, True)["step"]
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": w.name, "replays": replays, "ms_per_replay": round(ms, 4), "GBps": round(gbs, 2),
           "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_replay": nbytes,
           "byte_identical_to_host_split": identical, "status": int(d_status.item())}
    del x, out, host
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
