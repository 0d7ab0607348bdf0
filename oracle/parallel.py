"""Whole-workload oracle results, computed as independent oracle calls on threads.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` (full-size parity) and by the
CPU-baseline leg of ``bench.py``; nothing on the product path imports it.

The rowwise output of a row depends only on that row (its amax and its
16-element blocks), and the columnwise output of one column of one expert
depends only on that column's rows within the expert (the per-token and
per-column definitions of the row-scaled NVFP4 cast: "Implement per-token
NVFP4 fprop recipe", TransformerEngine PR 2931, Description; "[PyTorch]
Enable NVFP4 row-scaled (per-token) backward for GroupedLinear",
TransformerEngine PR 3324, Greptile Summary).  So one oracle call on the whole
buffer equals the concatenation of oracle calls on row ranges (rowwise
direction) and on column ranges of each expert (columnwise direction);
``tests/test_cpu_baseline.py`` checks that equality byte for byte.  The calls
go through ctypes, which releases the GIL, so a thread pool runs them in
parallel.  The arithmetic is entirely the C oracle's.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import oracle as O

ROWS_PER_TASK = 1024
COLS_PER_TASK = 1024
# worker threads: the host CPUs this process may run on, at most 16 (a
# one-GPU share of the GPU host's cores)
MAX_THREADS = 16


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(MAX_THREADS, n))


def tasks(splits, k: int, rowwise: bool, columnwise: bool,
          rows_per_task: int = ROWS_PER_TASK, cols_per_task: int = COLS_PER_TASK):
    """Independent pieces of one grouped call: ("row", r0, r1) and
    ("col", e, lo, hi, c0, c1), largest first.  Row ranges are whole 128-row
    groups (the oracle takes splits in 128-row units)."""
    if rows_per_task % 128:
        raise ValueError("rows_per_task must be a multiple of 128")
    sp = [int(v) for v in splits]
    offs = np.concatenate([[0], np.cumsum(sp)]).astype(np.int64)
    out = []
    if rowwise:
        total = int(offs[-1])
        out += [("row", r, min(r + rows_per_task, total)) for r in range(0, total, rows_per_task)]
    if columnwise:
        for e, m in enumerate(sp):
            lo, hi = int(offs[e]), int(offs[e + 1])
            if m:
                out += [("col", e, lo, hi, c, min(c + cols_per_task, k)) for c in range(0, k, cols_per_task)]
            else:  # an expert without rows: the oracle's call gives its (zero) column amax
                out.append(("col", e, lo, lo, 0, k))
    size = lambda t: (t[2] - t[1]) * k if t[0] == "row" else (t[3] - t[2]) * (t[5] - t[4])
    out.sort(key=size, reverse=True)
    return out


def alloc(sum_m: int, k: int, num_experts: int, rowwise: bool, columnwise: bool) -> dict:
    res = {"row_amax": None, "col_amax": None, "row_data": None, "row_scale": None,
           "col_data": None, "col_scale": None}
    if rowwise:
        res["row_amax"] = np.empty(sum_m, np.float32)
        res["row_data"] = np.empty((sum_m, k // 2), np.uint8)
        res["row_scale"] = np.empty((sum_m, k // 16), np.uint8)
    if columnwise:
        res["col_amax"] = np.empty(num_experts * k, np.float32)
        res["col_data"] = np.empty(sum_m * k // 2, np.uint8)
        res["col_scale"] = np.empty(sum_m * k // 16, np.uint8)
    return res


def _call(x, splits, rowwise, columnwise, four_over_six, amax=None):
    """The oracle on one piece: amax + cast, or (with ``amax`` = the piece's
    (row_amax, col_amax) slices of precomputed vectors) the cast alone."""
    if amax is None:
        if four_over_six is None:
            return O.group_quantize(x, splits, rowwise, columnwise)
        bound, err_mode = four_over_six
        return O.group_quantize_4o6(x, splits, bound, err_mode, rowwise, columnwise)
    ra, ca = amax
    if four_over_six is None:
        rd, rs, cd, cs = O.group_cast(x, splits, ra, ca, rowwise, columnwise)
    else:
        rd, rs, cd, cs = O.group_cast_4o6(x, splits, ra, ca, four_over_six[0], four_over_six[1], rowwise, columnwise)
    return {"row_amax": ra, "col_amax": ca, "row_data": rd, "row_scale": rs, "col_data": cd, "col_scale": cs}


def run_task(x: np.ndarray, k: int, task, res: dict, four_over_six=None, amax=None) -> None:
    """One oracle call; its bytes go to their place in the whole outputs.
    ``amax`` = whole precomputed (row_amax, col_amax) vectors (per-tensor
    scaling), sliced for the piece; otherwise the piece computes its own."""
    if task[0] == "row":
        _, r0, r1 = task
        piece = None if amax is None else (amax[0][r0:r1], None)
        part = _call(x[r0:r1], [r1 - r0], True, False, four_over_six, piece)
        res["row_amax"][r0:r1] = part["row_amax"]
        res["row_data"][r0:r1] = part["row_data"]
        res["row_scale"][r0:r1] = part["row_scale"]
    else:
        _, e, lo, hi, c0, c1 = task
        m = hi - lo
        xs = np.ascontiguousarray(x[lo:hi, c0:c1])
        piece = None if amax is None else (None, amax[1][e * k + c0:e * k + c1])
        part = _call(xs, [m], False, True, four_over_six, piece)
        res["col_amax"][e * k + c0:e * k + c1] = part["col_amax"]
        res["col_data"][k * lo // 2 + c0 * (m // 2):k * lo // 2 + c1 * (m // 2)] = part["col_data"]
        res["col_scale"][k * lo // 16 + c0 * (m // 16):k * lo // 16 + c1 * (m // 16)] = part["col_scale"]


def group_quantize(x: np.ndarray, splits, rowwise: bool = True, columnwise: bool = True,
                   threads: int | None = None, rows_per_task: int = ROWS_PER_TASK,
                   cols_per_task: int = COLS_PER_TASK, four_over_six=None, row_scaled: bool = True) -> dict:
    """The oracle's amax + cast of the whole packed buffer ``x`` (bf16 bits,
    (sum_m, k)), as one dict of numpy arrays (None for a direction not asked
    for).  ``four_over_six = (bound, err_mode)`` runs the oracle's
    four-over-six cast instead of the plain one (the pieces are independent
    in the same way: a block's choice depends only on its line).
    ``row_scaled=False``: the per-tensor amax (every line of an expert takes
    the expert's max |x|) is computed first, in one oracle call, and each
    piece casts with its slice of it."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sum_m, k = x.shape
    sp = [int(v) for v in splits]
    if sum(sp) != sum_m:
        raise ValueError("splits must sum to the row count")
    res = alloc(sum_m, k, len(sp), rowwise, columnwise)
    work = tasks(sp, k, rowwise, columnwise, rows_per_task, cols_per_task)
    amax = None
    if not row_scaled:
        ra, ca = O.group_amax_tensor(x, sp, True, True)
        amax = (ra, ca)
    n = threads or default_threads()
    if n == 1:
        for t in work:
            run_task(x, k, t, res, four_over_six, amax)
    else:
        with ThreadPoolExecutor(max_workers=n) as pool:
            for f in [pool.submit(run_task, x, k, t, res, four_over_six, amax) for t in work]:
                f.result()
    return res
