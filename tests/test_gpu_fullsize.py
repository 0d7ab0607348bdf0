"""The full-size workloads, in the launch configuration the benchmark times.

The rowwise-only outlier workload (8 experts, K=2048, sum_M=8192) is compared
with the oracle element by element.  The DeepSeek-V3-style expert share
(32 experts, K=7168, sum_M=65536), the down-projection input (64 experts,
K=2048, sum_M=131072) and the graph-replay workload are compared on sampled
rows and (expert, column) lines that the oracle computes one at a time, and
on properties of every element: each amax equals torch's exact max of |x|,
row and column amax agree per expert, zero-row experts give 0, guard bands
are intact.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import (alloc, assert_equal_outputs, assert_guards, first_mismatch, log, run_host_split,
                         tensors, to_device, to_numpy)

pytestmark = pytest.mark.gpu


def check_amax_everywhere(x_dev, splits, gpu):
    """Every amax element against torch's max of |x| (max is exact)."""
    a = x_dev.view(torch.bfloat16).abs()
    if "row_amax" in gpu:
        ref = a.amax(dim=1).float().cpu().numpy() if a.shape[0] else np.zeros(0, np.float32)
        assert first_mismatch(gpu["row_amax"], ref) is None
    if "col_amax" in gpu:
        k = a.shape[1]
        r0 = 0
        for e, m in enumerate(splits):
            seg = gpu["col_amax"][e * k:(e + 1) * k]
            if m == 0:
                assert (seg == 0).all()
            else:
                ref = a[r0:r0 + m].amax(dim=0).float().cpu().numpy()
                assert first_mismatch(seg, ref) is None, e
                if "row_amax" in gpu:
                    assert seg.max() == gpu["row_amax"][r0:r0 + m].max()
            r0 += m


def check_sampled(w, gpu, seed, n_rows=256, n_lines=160):
    rng = np.random.default_rng(seed)
    k = w.k
    offs = np.concatenate([[0], np.cumsum(w.splits)])
    if "row_data" in gpu:
        rows = set(rng.integers(0, w.sum_m, n_rows).tolist())
        for e in range(w.num_experts):
            if w.splits[e]:
                rows |= {int(offs[e]), int(offs[e + 1] - 1)}
        for r in sorted(rows):
            A = O.row_amax(w.x, r)
            assert gpu["row_amax"][r] == A, r
            d, s = O.cast_row(w.x, r, A)
            assert (gpu["row_data"][r] == d).all(), f"row {r}"
            assert (gpu["row_scale"][r] == s).all(), f"row scale {r}"
    if "col_data" in gpu:
        live = [e for e in range(w.num_experts) if w.splits[e]]
        lines = {(int(rng.choice(live)), int(rng.integers(0, k))) for _ in range(n_lines)}
        lines |= {(live[0], 0), (live[-1], k - 1), (int(np.argmax(w.splits)), k // 2)}
        for e, c in sorted(lines):
            r0, m = int(offs[e]), int(w.splits[e])
            A = O.col_amax(w.x, c, r0, m)
            assert gpu["col_amax"][e * k + c] == A, (e, c)
            d, s = O.cast_col(w.x, c, r0, m, A)
            got_d = gpu["col_data"][k * r0 // 2 + c * (m // 2): k * r0 // 2 + (c + 1) * (m // 2)]
            got_s = gpu["col_scale"][k * r0 // 16 + c * (m // 16): k * r0 // 16 + (c + 1) * (m // 16)]
            assert (got_d == d).all(), f"col line e={e} c={c}"
            assert (got_s == s).all(), f"col scale e={e} c={c}"


def test_outliers_rowwise_full_elementwise():
    w = synth.outliers()
    log(f"{w.name} splits={w.splits.tolist()}")
    x = to_device(w.x)
    out = run_host_split(x, list(map(int, w.splits)), True, False, entry="quantize")
    assert_guards(out)
    gpu = to_numpy(out)
    ref = O.group_quantize(w.x, w.splits, True, False)
    assert_equal_outputs(gpu, ref, ["row_amax", "row_data", "row_scale"])
    # and via the two separate calls
    out2 = to_numpy(run_host_split(x, list(map(int, w.splits)), True, False))
    assert_equal_outputs(out2, ref, ["row_amax", "row_data", "row_scale"])


@pytest.mark.parametrize("make", [synth.deepseek_share, synth.down_proj])
def test_large_both_directions_sampled(make):
    w = make()
    splits = list(map(int, w.splits))
    log(f"{w.name} splits={splits}")
    x = to_device(w.x)
    out = run_host_split(x, splits, True, True)
    assert_guards(out)
    gpu = to_numpy(out)
    check_amax_everywhere(x, splits, gpu)
    check_sampled(w, gpu, seed=7)
    del out
    # the one-call entry produces the same bytes
    log(f"{w.name} quantize entry")
    gpu2 = to_numpy(run_host_split(x, splits, True, True, entry="quantize"))
    assert_equal_outputs(gpu2, gpu)


def test_graph_replay_expert_share_shapes():
    # expert-share shapes, gradient-like values; capture once, replay with
    # new routing; every replay equals the host-split path byte for byte, and
    # sampled lines equal the oracle on the first and last replays
    w = synth.graph_replay()
    E, cap, k = w.num_experts, w.sum_m, w.k
    log(f"{w.name} capture")
    x = to_device(w.x)
    out = alloc(cap, k, E, True, True)
    t = tensors(out)
    d_offs = torch.tensor(B.offsets_from_splits(synth.replay_splits(0)), dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.nvfp4_group_quantize_graphsafe(x, E, d_offs, d_status, **t)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.nvfp4_group_quantize_graphsafe(x, E, d_offs, d_status, **t)
    for i in (0, 1, 2, 3):
        splits = [int(v) for v in synth.replay_splits(i)]
        log(f"replay {i} splits={splits}")
        d_offs.copy_(torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        got = to_numpy(out)
        host = to_numpy(run_host_split(x, splits))
        assert_equal_outputs(got, host)
        if i in (0, 3):
            wi = synth.Workload("replay", w.x, np.array(splits, np.int64))
            check_sampled(wi, got, seed=100 + i, n_rows=128, n_lines=96)
            check_amax_everywhere(x, splits, got)
        del host
    assert int(d_status.item()) == 0
    assert_guards(out)
