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

``flushed_step`` times the same steps with a 512 MB read before each
(outside the events), so that the 256 MB memory-side cache holds nothing of
the step's data; ``hbm_ceiling`` times a plain 1 GiB device copy in the same
process, the practical rate of a stream of reads and writes; ``cpu_baseline``
is the CPU oracle on a bounded sample, timed before the process touches the
GPU.

On workloads with both directions the JSON line also carries ``next_rows``:
the grouped MXFP4 cast of the same input (one read of x, both MXFP4 outputs
written), the rowwise / columnwise NVFP4 dequant of the step's outputs
(codes, scales and line amax read once, fp32 written), and the row-scaled
grouped GEMM (forward and weight gradient, MFMA-bound, TFLOP/s against the
fp16 MFMA peak), each timed with HIP events over repeated launches; beside
the GEMM, torch.matmul (hipBLASLt) in fp16 on operands of the same shapes,
for context.
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
METRIC = "grouped NVFP4 amax+cast HBM GB/s (bytes in+out) and % of MI355X peak BW"
# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, per workload
TRAFFIC_FILES = {"deepseek_share": "profiles/group_cast_kernel-deepseek_share_e32_k7168_m65536.md",
                 "down_proj": "profiles/group_cast_kernel-down_proj_e64_k2048_m131072.md"}


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


_SAMPLE_X = None  # the sample's rows, inherited by the forked oracle workers
_TASK_ROWS = 1024  # rows per rowwise task
_TASK_COLS = 1024  # columns per columnwise task


def _oracle_task(task) -> None:
    rowwise, lo, hi, c0, c1 = task
    from oracle import oracle as O
    x = _SAMPLE_X[lo:hi] if rowwise else np.ascontiguousarray(_SAMPLE_X[lo:hi, c0:c1])
    O.group_quantize(x, [hi - lo], rowwise, not rowwise)


def cpu_baseline(w, target_rows: int = 16384, max_workers: int = 16) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole experts (in expert order, skipping any that would overshoot) up to
    ``target_rows`` rows, both directions.  Timed on one thread (one call),
    then on the host's cores (at most ``max_workers`` forked processes) as
    independent oracle calls: the rowwise direction on row ranges and the
    columnwise direction on column ranges of each expert (rows are
    independent in the rowwise output and columns in the columnwise one, so
    together the calls produce the same bytes as the single call).  Runs
    before the process touches the GPU, so that forking is safe."""
    global _SAMPLE_X
    import multiprocessing
    from oracle import oracle as O
    offs = np.concatenate([[0], np.cumsum(w.splits)])
    chosen, rows = [], 0
    for e, m in enumerate(w.splits):
        if m and rows + int(m) <= target_rows:
            chosen.append(e)
            rows += int(m)
    xs = np.concatenate([w.x[offs[e]:offs[e + 1]] for e in chosen])
    sp = [int(w.splits[e]) for e in chosen]
    t0 = time.perf_counter()
    O.group_quantize(xs, sp, w.rowwise, w.columnwise)
    dt1 = time.perf_counter() - t0
    _SAMPLE_X = xs
    so = np.concatenate([[0], np.cumsum(sp)]).astype(int)
    tasks = []
    for i in range(len(sp)):
        lo, hi = int(so[i]), int(so[i + 1])
        if w.rowwise:
            tasks += [(True, r, min(r + _TASK_ROWS, hi), 0, w.k) for r in range(lo, hi, _TASK_ROWS)]
        if w.columnwise:
            tasks += [(False, lo, hi, c, min(c + _TASK_COLS, w.k)) for c in range(0, w.k, _TASK_COLS)]
    tasks.sort(key=lambda t: (t[2] - t[1]) * (t[4] - t[3]), reverse=True)
    workers = max(1, min(max_workers, os.cpu_count() or 1, len(tasks)))
    with multiprocessing.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        list(pool.imap_unordered(_oracle_task, tasks))
        dtn = time.perf_counter() - t0
    _SAMPLE_X = None
    b = algorithmic_bytes(rows, w.k, len(sp), w.rowwise, w.columnwise)["step"]
    return {"value": round(b / dtn / 1e9, 5), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(sp)} whole experts, {rows} of {w.sum_m} rows x K={w.k} (both directions), "
                      f"C oracle: {len(tasks)} row-range / column-range calls over {workers} processes "
                      f"{dtn:.2f} s, one call on one thread {dt1:.2f} s",
            "value_one_thread": round(b / dt1 / 1e9, 5)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed steps for this long before the warmup steps: the GPU's clocks ramp up over "
                         "the first tens of milliseconds of load on a fresh box (0: skip)")
    ap.add_argument("--workload", default="deepseek_share",
                    choices=["deepseek_share", "down_proj", "outliers", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-replays", type=int, default=100)
    ap.add_argument("--next-rows", type=int, default=20,
                    help="launches timed for each of the MXFP4 cast and the two dequants (0: skip)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="also time the steps with a read of this many MB before each (outside the timed "
                         "events), so that no input or output is left in the 256 MB memory-side cache (0: skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (3 times, untimed) so that a "
                         "rocprofv3 --pmc run can scale FETCH_SIZE / WRITE_SIZE by a copy of known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    from nvfp4_block_scaled_group_amd import synth

    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    w = synth.CONFIGS[args.workload]()
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (before any GPU use)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)

    import torch
    from nvfp4_block_scaled_group_amd import binding as B

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    splits = [int(v) for v in w.splits]
    E, k, m = w.num_experts, w.k, w.sum_m
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    out = B.alloc_outputs(m, k, E, w.rowwise, w.columnwise, device=dev)
    nbytes = algorithmic_bytes(m, k, E, w.rowwise, w.columnwise)

    fused = w.rowwise and not w.columnwise
    # small inputs with a columnwise output: the library's one-launch path
    small = w.columnwise and max(splits) * k <= B.SMALL_MAX_EXPERT_ELEMS and k <= B.SMALL_MAX_K

    tev = TimingEvents(torch)

    def step(ev=None):
        if ev is not None:
            tev.record(ev[0])
        if fused or small:
            # rowwise only: one pass (row amax and cast together); small
            # inputs: one launch, one work-group per expert
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

    print(f"[bench] settle {args.settle_ms:.0f} ms, warmup {args.warmup}", file=sys.stderr, flush=True)
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[tev.new() for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    first_ms = float(np.mean([tev.elapsed_ms(e[0], e[1]) for e in events]))
    second_ms = float(np.mean([tev.elapsed_ms(e[1], e[2]) for e in events]))
    ms_per_step = wall * 1e3 / args.steps
    value = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    if fused or small:
        dom_name, dom_ms = ("group_quantize_rowwise_kernel", first_ms) if fused else \
            ("group_quantize_small_kernel", first_ms)
        dom_bytes = nbytes["fused_kernel"] if fused else nbytes["step"]
        kernels = {dom_name: {"avg_us": round(dom_ms * 1e3, 2), "GBps": round(dom_bytes / dom_ms / 1e6, 2)}}
    else:
        dom_name, dom_ms, dom_bytes = "group_cast_kernel", second_ms, nbytes["cast_kernel"]
        amax_name = "group_amax_rows_kernel" if k <= 2048 else "group_amax_kernel"
        kernels = {f"amax (init + {amax_name})": {"avg_us": round(first_ms * 1e3, 2),
                                                  "GBps": round(nbytes["amax_kernel"] / first_ms / 1e6, 2)},
                   "group_cast_kernel": {"avg_us": round(second_ms * 1e3, 2),
                                         "GBps": round(nbytes["cast_kernel"] / second_ms / 1e6, 2)}}
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9

    # HBM bytes per launch of the cast kernel from the committed FETCH_SIZE /
    # WRITE_SIZE summary, only while the HIP source is the one it was taken on
    from nvfp4_block_scaled_group_amd import profiling
    traffic_file = TRAFFIC_FILES.get(args.workload)
    traffic = profiling.load_traffic(os.path.join(ROOT, traffic_file), dom_name) if traffic_file else None

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "num_experts": E, "k": k, "sum_m": m,
                   "directions": "+".join(d for d, on in (("rowwise", w.rowwise), ("columnwise", w.columnwise))
                                          if on),
                   "entry": ("nvfp4_group_quantize (host splits, fused rowwise pass)" if fused
                             else "nvfp4_group_quantize (host splits, one launch for a small input)" if small
                             else "nvfp4_group_amax + nvfp4_group_cast (host splits)"),
                   "algorithmic_bytes_per_step": nbytes["step"],
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(dom_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_source": traffic_file if traffic else None,
                     "avg_us": round(dom_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": dom_bytes},
        "kernels": kernels,
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
        f_ms = float(np.mean([tev.elapsed_ms(e[0], e[2]) for e in fev]))
        result["flushed_step"] = {"flush_mb": args.flush_mb, "steps": args.steps,
                                  "ms_per_step": round(f_ms, 4),
                                  "GBps": round(nbytes["step"] / (f_ms * 1e-3) / 1e9, 2),
                                  "unflushed_event_ms_per_step": round(first_ms + second_ms, 4)}
        del flush

    result["hbm_ceiling"] = copy_ceiling(torch, tev, dev)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if w.rowwise and w.columnwise and args.next_rows > 0:
        result["next_rows"] = next_rows(B, torch, tev, x, splits, out, E, k, m, args.next_rows)

    if args.workload == "deepseek_share" and args.graph_replays > 0:
        result["graph_replay"] = graph_replay(B, synth, torch, tev, dev, args.graph_replays)

    if cpu is not None:
        result["cpu_baseline"] = cpu
    tev.close()
    print(json.dumps(result), flush=True)


def copy_ceiling(torch, tev, dev, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """Context for roofline.frac: a plain device-to-device copy of 1 GiB on
    the same GPU in the same process (bytes read + written over its time,
    HIP events on the same stream), the rate a stream that mixes reads and
    writes reaches on this memory system."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(tev.new(), tev.new()) for _ in range(reps)]
    for e0, e1 in evs:
        tev.record(e0)
        dst.copy_(src)
        tev.record(e1)
    torch.cuda.synchronize()
    ms = float(np.mean([tev.elapsed_ms(a, b) for a, b in evs]))
    del src, dst
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"kind": "device copy, 1 GiB read + 1 GiB written", "avg_us": round(ms * 1e3, 2),
            "GBps": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def next_rows(B, torch, tev, x, splits, out, E: int, k: int, m: int, reps: int) -> dict:
    """MXFP4 cast of the step's input and NVFP4 dequant of its outputs."""
    print("[bench] MXFP4 cast and dequant", file=sys.stderr, flush=True)
    N = m * k

    def timed(fn):
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
    mx = B.alloc_mx_outputs(m, k, device=x.device)
    ms = timed(lambda: B.mxfp4_group_cast(x, splits, **mx))
    res["mxfp4_group_cast"] = entry("mxfp4_group_cast_kernel", ms, 2 * N + 2 * (N // 2 + N // 32))
    del mx
    deq = torch.empty(N, dtype=torch.float32, device=x.device)
    ms = timed(lambda: B.nvfp4_group_dequant_rowwise(out["row_data"], out["row_scale"], out["row_amax"],
                                                      deq.view(m, k)))
    res["nvfp4_group_dequant_rowwise"] = entry("dequant_kernel", ms, N // 2 + N // 16 + 4 * m + 4 * N)
    ms = timed(lambda: B.nvfp4_group_dequant_columnwise(out["col_data"], out["col_scale"], out["col_amax"],
                                                         splits, k, deq))
    res["nvfp4_group_dequant_columnwise"] = entry("dequant_kernel", ms, N // 2 + N // 16 + 4 * E * k + 4 * N)
    del deq
    res.update(gemm_rows(B, torch, timed, out, splits, E, k, m))
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
    one hipGraph capture of amax + cast, replayed with new routing written to
    the device offsets before each replay (the offset copy is outside the
    timed launches)."""
    print("[bench] graph replay workload", file=sys.stderr, flush=True)
    w = synth.graph_replay()
    E, k, m = w.num_experts, w.k, w.sum_m
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    out = B.alloc_outputs(m, k, E, True, True, device=dev)
    routes = [torch.tensor(B.offsets_from_splits(synth.replay_splits(i)), dtype=torch.int32).pin_memory()
              for i in range(replays)]
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
    times = []
    for i in range(replays):
        d_offs.copy_(routes[i], non_blocking=True)
        e0, e1 = tev.new(), tev.new()
        tev.record(e0)
        g.replay()
        tev.record(e1)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([tev.elapsed_ms(a, b) for a, b in times]))
    nbytes = algorithmic_bytes(m, k, E, True, True)["step"]
    return {"workload": w.name, "replays": replays, "ms_per_replay": round(ms, 4),
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 2), "status": int(d_status.item())}


if __name__ == "__main__":
    main()
