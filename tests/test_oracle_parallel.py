"""The threaded whole-workload oracle (row ranges and per-expert column
ranges as independent oracle calls) gives exactly the bytes of one oracle
call, including experts without rows and ragged last pieces."""
import numpy as np
import pytest

from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O
from oracle import parallel as OP

KEYS = ("row_amax", "col_amax", "row_data", "row_scale", "col_data", "col_scale")


@pytest.mark.parametrize("rowwise,columnwise", [(True, True), (True, False), (False, True)])
def test_parallel_equals_one_call(rowwise, columnwise):
    w = synth.random_case(21, [384, 0, 128, 640, 0, 256], 272, "rowscale")
    ref = O.group_quantize(w.x, w.splits, rowwise, columnwise)
    got = OP.group_quantize(w.x, w.splits, rowwise, columnwise, threads=4, rows_per_task=256,
                            cols_per_task=48)
    for key in KEYS:
        if ref[key] is None:
            assert got[key] is None
            continue
        a, b = np.asarray(got[key]), np.asarray(ref[key])
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        assert np.array_equal(a.reshape(-1), b.reshape(-1)), key


def test_tasks_cover_every_row_and_column_once():
    sp, k = [256, 0, 1280], 2064
    work = OP.tasks(sp, k, True, True, rows_per_task=384, cols_per_task=1000)
    rows = sorted((t[1], t[2]) for t in work if t[0] == "row")
    assert rows[0][0] == 0 and rows[-1][1] == sum(sp)
    assert all(a[1] == b[0] for a, b in zip(rows, rows[1:]))
    for e, m in enumerate(sp):
        cols = sorted((t[4], t[5]) for t in work if t[0] == "col" and t[1] == e)
        assert cols[0][0] == 0 and cols[-1][1] == k
        assert all(a[1] == b[0] for a, b in zip(cols, cols[1:]))


def test_default_threads_bounded():
    assert 1 <= OP.default_threads() <= OP.MAX_THREADS


@pytest.mark.parametrize("bound,mode", [(256, 0), (448, 1)])
def test_parallel_four_over_six_equals_one_call(bound, mode):
    w = synth.random_case(23, [256, 0, 384, 128], 96, "rowscale")
    ref = O.group_quantize_4o6(w.x, w.splits, bound, mode)
    got = OP.group_quantize(w.x, w.splits, threads=3, rows_per_task=128, cols_per_task=32,
                            four_over_six=(bound, mode))
    for key in KEYS:
        a, b = np.asarray(got[key]), np.asarray(ref[key])
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        assert np.array_equal(a.reshape(-1), b.reshape(-1)), key


@pytest.mark.parametrize("four_over_six", [None, (256, 0), (448, 1)])
def test_parallel_per_tensor_equals_one_call(four_over_six):
    """Per-tensor scaling (row_scaled False): the pieces cast with slices of
    the expert amax vectors computed once, giving the single call's bytes."""
    w = synth.random_case(23, [256, 0, 384, 128], 96, "rowscale")
    sp = [int(v) for v in w.splits]
    if four_over_six is None:
        ref = O.group_quantize(w.x, sp, row_scaled=False)
    else:
        ref = O.group_quantize_4o6(w.x, sp, four_over_six[0], four_over_six[1], row_scaled=False)
    got = OP.group_quantize(w.x, sp, threads=3, rows_per_task=128, cols_per_task=32, four_over_six=four_over_six,
                            row_scaled=False)
    for key in ref:
        assert np.array_equal(np.asarray(got[key]).reshape(-1), np.asarray(ref[key]).reshape(-1)), key
