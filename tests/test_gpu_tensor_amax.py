"""The per-tensor amax (row scaling off: every line of an expert takes the
expert's max |x|) on the GPU, through the C ABI, against the oracle: the
amax vectors bit for bit, the plain and the four-over-six casts consuming
them byte for byte (small, ragged and full-size workloads), and the
graph-safe form under partial routing."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O
from oracle import parallel as OP

from gpu_helpers import alloc, assert_equal_outputs, assert_guards, log, tensors, to_device, to_numpy

pytestmark = pytest.mark.gpu

CASES = [
    ([128, 0, 256, 128], 272, "rowscale", 61),
    ([384, 128], 48, "outliers", 62),
    ([0, 256, 0], 784, "normal", 63),
    ([128] * 9, 96, "student", 64),
]


def run(w, cast, rowwise=True, columnwise=True, **knobs):
    splits = list(map(int, w.splits))
    x = to_device(w.x)
    out = alloc(w.sum_m, w.k, len(splits), rowwise, columnwise)
    t = tensors(out)
    B.nvfp4_group_amax_tensor(x, splits, t["row_amax"], t["col_amax"])
    if cast == "plain":
        B.nvfp4_group_cast(x, splits, **t)
    elif cast == "4o6":
        B.nvfp4_group_cast_4over6(x, splits, **t, **knobs)
    torch.cuda.synchronize()
    assert_guards(out)
    return to_numpy(out)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_amax_vectors(case):
    splits, k, dist, seed = CASES[case]
    w = synth.random_case(seed, splits, k, dist)
    log(f"tensor amax {w.name} splits={splits} k={k}")
    for rowwise, columnwise in ((True, True), (True, False), (False, True)):
        gpu = run(w, None, rowwise, columnwise)
        ra, ca = O.group_amax_tensor(w.x, splits, rowwise, columnwise)
        if rowwise:
            assert np.array_equal(gpu["row_amax"].view(np.uint32), ra.view(np.uint32))
        if columnwise:
            assert np.array_equal(gpu["col_amax"].view(np.uint32), ca.view(np.uint32))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_plain_cast_per_tensor(case):
    splits, k, dist, seed = CASES[case]
    w = synth.random_case(seed, splits, k, dist)
    log(f"per-tensor plain cast {w.name}")
    assert_equal_outputs(run(w, "plain"), O.group_quantize(w.x, splits, row_scaled=False))


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("bound,mode", [(256, B.ERR_MSE), (448, B.ERR_MAE), (3, B.ERR_MSE)])
def test_four_over_six_per_tensor(case, bound, mode):
    splits, k, dist, seed = CASES[case]
    w = synth.random_case(seed, splits, k, dist)
    log(f"per-tensor four-over-six {w.name} bound={bound} mode={mode}")
    gpu = run(w, "4o6", scale_bound=bound, err_mode=mode)
    assert_equal_outputs(gpu, O.group_quantize_4o6(w.x, splits, bound, mode, row_scaled=False))


def test_graphsafe_partial_routing():
    """Capacity 1024 rows, routed 640: the routed lines equal the host-split
    call's, and rows at or beyond the routed total keep their prefill."""
    k, cap, splits = 272, 1024, [256, 0, 384]
    w = synth.random_case(65, [cap], k, "rowscale")
    x = to_device(w.x)
    routed = sum(splits)
    offs = torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    o = alloc(cap, k, len(splits), True, True)
    for g in o.values():
        g.t.view(torch.uint8).fill_(0x5A)
    t = tensors(o)
    B.nvfp4_group_amax_tensor_graphsafe(x, len(splits), offs, status, t["row_amax"], t["col_amax"])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_guards(o)
    ra, ca = O.group_amax_tensor(w.x[:routed], splits)
    got = to_numpy(o)
    assert np.array_equal(got["row_amax"][:routed].view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(got["col_amax"].view(np.uint32), ca.view(np.uint32))
    assert (got["row_amax"][routed:].view(np.uint8) == 0x5A).all()


def test_full_size_four_over_six_per_tensor():
    """The expert-share workload (65536 x 7168, 32 experts), both directions,
    per-tensor four-over-six cast: every amax, data byte and scale byte."""
    w = synth.deepseek_share()
    splits = list(map(int, w.splits))
    log("per-tensor four-over-six, expert-share workload: GPU")
    x = to_device(w.x)
    out = B.alloc_outputs(w.sum_m, w.k, len(splits))
    B.nvfp4_group_amax_tensor(x, splits, out["row_amax"], out["col_amax"])
    B.nvfp4_group_cast_4over6(x, splits, **out, scale_bound=256, err_mode=B.ERR_MSE)
    torch.cuda.synchronize()
    gpu = {key: t.cpu().numpy() for key, t in out.items()}
    del x, out
    log("per-tensor four-over-six, expert-share workload: oracle")
    ref = OP.group_quantize(w.x, splits, True, True, four_over_six=(256, B.ERR_MSE), row_scaled=False)
    for key in ("row_amax", "col_amax"):
        assert np.array_equal(gpu[key].view(np.uint32), ref[key].view(np.uint32)), key
    for key in ("row_data", "row_scale", "col_data", "col_scale"):
        bad = np.count_nonzero(gpu[key].reshape(-1) != ref[key].reshape(-1))
        assert bad == 0, f"{key}: {bad} mismatching bytes"
