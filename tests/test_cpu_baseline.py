"""The benchmark's CPU baseline (and the full-size parity tests) split one
oracle call into independent calls: the rowwise direction on row ranges and
the columnwise direction on column ranges of each expert.  Rows are independent in the rowwise output
(each row has its own amax and blocks) and columns in the columnwise output
(each column of an expert is its own line), so the pieces must reproduce the
single call's bytes; this is checked here, and the baseline is run once on
the tiny workload."""
import numpy as np

import bench
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O


def test_split_calls_reproduce_the_single_call():
    w = synth.random_case(11, [256, 0, 384, 128], 96, "rowscale")
    x, sp, k = w.x, [int(v) for v in w.splits], w.k
    ref = O.group_quantize(x, sp)
    offs = np.concatenate([[0], np.cumsum(sp)]).astype(int)
    for e, m in enumerate(sp):
        lo, hi = offs[e], offs[e + 1]
        for r in range(lo, hi, 128):  # row ranges, rowwise only
            part = O.group_quantize(x[r:r + 128], [128], True, False)
            assert np.array_equal(part["row_amax"], ref["row_amax"][r:r + 128])
            assert np.array_equal(part["row_data"], ref["row_data"][r:r + 128])
            assert np.array_equal(part["row_scale"], ref["row_scale"][r:r + 128])
        if m == 0:
            continue
        col_data = ref["col_data"][k * lo // 2: k * hi // 2].reshape(k, m // 2)
        col_scale = ref["col_scale"][k * lo // 16: k * hi // 16].reshape(k, m // 16)
        for c in range(0, k, 32):  # column ranges, columnwise only
            part = O.group_quantize(np.ascontiguousarray(x[lo:hi, c:c + 32]), [m], False, True)
            assert np.array_equal(part["col_amax"], ref["col_amax"][e * k + c: e * k + c + 32])
            assert np.array_equal(part["col_data"].reshape(32, m // 2), col_data[c:c + 32])
            assert np.array_equal(part["col_scale"].reshape(32, m // 16), col_scale[c:c + 32])


def test_cpu_baseline_runs_on_the_tiny_workload():
    r = bench.cpu_baseline(synth.tiny(), threads=2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["value_one_thread"] > 0 and r["cores"] == r["threads"] == 2
    assert r["nproc"] >= 1 and "whole workload" in r["sample"]
