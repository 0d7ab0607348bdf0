"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Inputs are compared element by element (every amax, FP4 byte and E4M3
scale, bit-exact), with guard bands around every output; the full-size
workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O
from oracle import parallel as OP

from gpu_helpers import (alloc, assert_equal_outputs, assert_guards, first_mismatch, log, run_host_split,
                         tensors, to_device, to_numpy)

pytestmark = pytest.mark.gpu


def oracle_ref(w, rowwise=True, columnwise=True):
    return O.group_quantize(w.x, w.splits, rowwise, columnwise)


def check_small(w, rowwise=True, columnwise=True, entry="two_calls"):
    log(f"{w.name} m={w.sum_m} k={w.k} splits={list(map(int, w.splits))} "
        f"row={rowwise} col={columnwise} entry={entry}")
    out = run_host_split(to_device(w.x), list(map(int, w.splits)), rowwise, columnwise, entry)
    assert_guards(out)
    gpu = to_numpy(out)
    ref = oracle_ref(w, rowwise, columnwise)
    assert_equal_outputs(gpu, ref)
    # dequantised cross-check: the oracle's dequant applied to the GPU bytes
    # against the oracle's dequant of its own bytes (max abs error <= 1e-6)
    if rowwise and w.sum_m:
        a = O.decode_rowwise(gpu["row_data"], gpu["row_scale"], gpu["row_amax"])
        b = O.decode_rowwise(ref["row_data"], ref["row_scale"], ref["row_amax"])
        assert np.abs(a.astype(np.float64) - b).max() <= 1e-6
    if columnwise and w.sum_m:
        a = O.decode_columnwise(gpu["col_data"], gpu["col_scale"], gpu["col_amax"], w.splits, w.k)
        b = O.decode_columnwise(ref["col_data"], ref["col_scale"], ref["col_amax"], w.splits, w.k)
        assert np.abs(a.astype(np.float64) - b).max() <= 1e-6
    return gpu


SMALL = [
    ([128, 0, 256, 128], 272, "normal", 31),       # 272 = 256 + 16: ragged column chunk
    ([384, 128], 48, "outliers", 32),
    ([256, 256, 0, 0, 512], 784, "outliers", 33),  # 784 = 3*256 + 16
    ([128, 128, 128], 16, "sparse", 34),           # all-zero blocks and rows
    ([640, 128], 2064, "rowscale", 35),
    ([0, 256, 128, 0], 512, "student", 36),        # gradient-like small values
    ([128] * 9, 96, "normal", 37),
]


def test_tiny_config_both_directions():
    check_small(synth.tiny())


def test_tiny_config_quantize_entry():
    check_small(synth.tiny(), entry="quantize")


@pytest.mark.parametrize("splits,k,dist,seed", SMALL)
def test_small_cases(splits, k, dist, seed):
    check_small(synth.random_case(seed, splits, k, dist))


@pytest.mark.parametrize("rowwise,columnwise", [(True, False), (False, True)])
def test_single_direction(rowwise, columnwise):
    w = synth.random_case(40, [256, 128, 0, 384], 336, "rowscale")
    check_small(w, rowwise, columnwise)
    check_small(w, rowwise, columnwise, entry="quantize")


def test_subnormal_and_tiny_values():
    # bf16 subnormals and tiny normals: line scales, block decode scales and
    # products in the fp32 denormal range, and the 1/d clamp.
    rng = np.random.default_rng(41)
    M, K = 384, 80
    v = rng.standard_normal((M, K)).astype(np.float32)
    row_exp = rng.integers(-133, -100, (M, 1)).astype(np.float32)
    v = v * np.exp2(row_exp)
    v[::7] *= np.float32(2.0 ** 60)          # some ordinary rows in between
    w = synth.Workload("tiny_values", synth.f32_to_bf16_bits(v), np.array([128, 256], np.int64))
    check_small(w)


def test_mixed_extremes_within_lines():
    # a huge outlier next to tiny values in the same line: most blocks get
    # subnormal or zero E4M3 scales
    rng = np.random.default_rng(42)
    M, K = 256, 64
    v = (rng.standard_normal((M, K)) * 1e-6).astype(np.float32)
    v[np.arange(M), rng.integers(0, K, M)] = np.float32(3e4)
    w = synth.Workload("extremes", synth.f32_to_bf16_bits(v), np.array([256], np.int64))
    check_small(w)


def test_closed_form_roundtrip_on_gpu():
    rng = np.random.default_rng(43)
    M, K = 384, 64
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    g = grid[rng.integers(0, 8, (M, K))] * rng.choice([-1.0, 1.0], (M, K))
    r, c = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    diag = (r % 16) == (c % 16)
    g[diag] = 6.0 * rng.choice([-1.0, 1.0], int(diag.sum()))
    xf = (g * 448.0 * 2.0 ** -7).astype(np.float32)
    w = synth.Workload("closed_form", synth.f32_to_bf16_bits(xf), np.array([128, 256], np.int64))
    gpu = check_small(w)
    back = O.decode_rowwise(gpu["row_data"], gpu["row_scale"], gpu["row_amax"])
    assert (back.view(np.uint32) == xf.view(np.uint32)).all()


def test_golden_row_on_gpu():
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_row_k64.txt")
    xs, exp = [], {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            if key == "x":
                xs += [int(v, 16) for v in vals]
            else:
                exp[key] = [int(v, 16) for v in vals]
    X = np.zeros((128, 64), np.uint16)
    X[0] = xs
    X[1:, 0] = 0x3F80  # other rows: a single 1.0
    w = synth.Workload("golden", X, np.array([128], np.int64))
    gpu = check_small(w)
    assert gpu["row_data"][0].tolist() == exp["data"]
    assert gpu["row_scale"][0].tolist() == exp["scale"]


def test_empty_input():
    log("empty input sum_m=0")
    x = torch.zeros((0, 64), dtype=torch.int16, device="cuda:0")
    out = run_host_split(x, [0, 0, 0], True, True)
    assert_guards(out)
    gpu = to_numpy(out)
    assert (gpu["col_amax"] == 0).all()


def test_deterministic():
    w = synth.random_case(44, [256, 0, 512], 528, "outliers")
    log("determinism")
    x = to_device(w.x)
    a = to_numpy(run_host_split(x, list(map(int, w.splits))))
    b = to_numpy(run_host_split(x, list(map(int, w.splits))))
    assert_equal_outputs(a, b)


# ----------------------------------------------------------- graph-safe path

def _graphsafe(x_dev, E, offs, m_cap, rowwise=True, columnwise=True, prefill=None, entry="two_calls"):
    k = x_dev.shape[1]
    out = alloc(m_cap, k, E, rowwise, columnwise)
    if prefill is not None:
        for g in out.values():
            g.t.view(torch.uint8).fill_(prefill)
    d_offs = torch.tensor(offs, dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    t = tensors(out)
    if entry == "two_calls":
        B.nvfp4_group_amax_graphsafe(x_dev, E, d_offs, d_status, t["row_amax"], t["col_amax"])
        B.nvfp4_group_cast_graphsafe(x_dev, E, d_offs, d_status, **t)
    else:
        B.nvfp4_group_quantize_graphsafe(x_dev, E, d_offs, d_status, **t)
    torch.cuda.synchronize()
    return out, int(d_status.item())


def test_graphsafe_matches_host_split():
    w = synth.random_case(45, [384, 0, 128, 640, 0, 256], 272, "rowscale")
    splits = list(map(int, w.splits))
    log("graph-safe vs host-split")
    x = to_device(w.x)
    host = to_numpy(run_host_split(x, splits))
    gs, status = _graphsafe(x, len(splits), B.offsets_from_splits(splits), w.sum_m)
    assert status == 0
    assert_guards(gs)
    assert_equal_outputs(to_numpy(gs), host)
    assert_equal_outputs(host, oracle_ref(w))


def test_graphsafe_leaves_rows_beyond_total_untouched():
    # buffers for 1024 rows, routing covers 640: rows 640.. keep their bytes
    rng = np.random.default_rng(46)
    cap, k = 1024, 96
    xf = rng.standard_normal((cap, k)).astype(np.float32)
    xb = synth.f32_to_bf16_bits(xf)
    splits = [256, 0, 384]
    log("graph-safe partial routing")
    x = to_device(xb)
    gs, status = _graphsafe(x, 3, B.offsets_from_splits(splits), cap, prefill=0x5A)
    assert status == 0
    assert_guards(gs)
    g = to_numpy(gs)
    tot = sum(splits)
    assert (g["row_amax"][tot:].view(np.uint32) == 0x5A5A5A5A).all()
    assert (g["row_data"][tot:] == 0x5A).all() and (g["row_scale"][tot:] == 0x5A).all()
    assert (g["col_data"][k * tot // 2:] == 0x5A).all() and (g["col_scale"][k * tot // 16:] == 0x5A).all()
    w = synth.Workload("partial", xb[:tot], np.array(splits, np.int64))
    ref = oracle_ref(w)
    assert first_mismatch(g["row_amax"][:tot], ref["row_amax"]) is None
    assert first_mismatch(g["row_data"][:tot], ref["row_data"]) is None
    assert first_mismatch(g["row_scale"][:tot], ref["row_scale"]) is None
    assert first_mismatch(g["col_amax"], ref["col_amax"]) is None
    assert first_mismatch(g["col_data"][:k * tot // 2], ref["col_data"]) is None
    assert first_mismatch(g["col_scale"][:k * tot // 16], ref["col_scale"]) is None


@pytest.mark.parametrize("offs,bits", [
    ([256, 128, 384], B.NVFP4G_DEV_NONMONO),
    ([256, 300, 384], B.NVFP4G_DEV_UNALIGNED),
    ([256, 384, 1280], B.NVFP4G_DEV_OVERFLOW),
    ([-128, 0, 128], B.NVFP4G_DEV_NONMONO),
])
def test_graphsafe_rejects_bad_device_routing(offs, bits):
    log(f"bad device routing {offs}")
    x = torch.zeros((1024, 32), dtype=torch.int16, device="cuda:0")
    gs, status = _graphsafe(x, 3, offs, 1024, prefill=0x33)
    assert status & bits
    assert_guards(gs)
    for key, g in to_numpy(gs).items():
        assert (g.view(np.uint8) == 0x33).all(), key


@pytest.mark.parametrize("E,cap,k", [
    (8, 2048, 400),   # the general path (zero-fill, amax, cast)
    (4, 256, 256),    # capacity * k at the one-launch limit: the small-input kernel
])
def test_graph_capture_replays_under_new_routing(E, cap, k):
    # one capture, replays with new routing written to the device offsets;
    # every replay equals the host-split path on that routing, byte for byte
    rng = np.random.default_rng(47)
    xb = synth.f32_to_bf16_bits((rng.standard_t(3.0, (cap, k)) * 1e-3).astype(np.float32))
    x = to_device(xb)
    out = alloc(cap, k, E, True, True)
    t = tensors(out)
    d_offs = torch.zeros(E, dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def routing(i):
        units = np.random.default_rng(100 + i).multinomial(cap // 128, np.full(E, 1.0 / E))
        return [int(u) * 128 for u in units]

    log("graph capture")
    d_offs.copy_(torch.tensor(B.offsets_from_splits(routing(0)), dtype=torch.int32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.nvfp4_group_quantize_graphsafe(x, E, d_offs, d_status, **t)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.nvfp4_group_quantize_graphsafe(x, E, d_offs, d_status, **t)
    for i in range(6):
        splits = routing(i)
        log(f"replay {i} splits={splits}")
        d_offs.copy_(torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        got = to_numpy(out)
        host = to_numpy(run_host_split(x, splits))
        assert_equal_outputs(got, host)
        if i in (0, 5):
            assert_equal_outputs(host, oracle_ref(synth.Workload("r", xb, np.array(splits, np.int64))))
    assert int(d_status.item()) == 0
    assert_guards(out)


# ------------------------------------------------------- more shapes / entries

# rows per tile of the whole-row amax (K <= 2048): 4 waves x 16 / 8 / 4 / 4
# rows for 1 / 2 / 3 / 4 column chunks of 512; its grid is min(rows/16, 512)
AMAX_ROW_TILE = {1: 64, 2: 32, 3: 16, 4: 16}


@pytest.mark.parametrize("k", [512, 528, 1040, 1552, 2032])
def test_amax_row_tiles_ragged_k_and_long_ranges(k):
    # K <= 2048 takes the amax that reads whole rows (1 - 4 column chunks per
    # lane).  Enough rows that every work-group walks at least 3 tiles (so the
    # next-tile prefetch and the column flush on an expert change inside a
    # range both run), with small experts so that ranges cross expert ends.
    nch = (k + 511) // 512
    tr = AMAX_ROW_TILE[nch]
    grid = 512
    rows = 3 * grid * tr + 128 * 5
    rng = np.random.default_rng(k)
    units, left = [], rows // 128
    while left:
        u = int(min(left, rng.integers(0, 4)))
        units.append(u)
        left -= u
    splits = [u * 128 for u in units]
    tiles = rows // tr
    assert min(rows // 16, 512) == grid and tiles >= 3 * grid, (tiles, grid)
    assert sum(1 for u in units if u == 0) >= 1 and len(units) > tiles // (3 * 16)
    w = synth.random_case(70 + k, splits, k, "rowscale")
    log(f"k={k} rows={rows} experts={len(splits)} tiles={tiles} grid={grid}")
    out = run_host_split(to_device(w.x), splits)
    assert_guards(out)
    assert_equal_outputs(to_numpy(out), OP.group_quantize(w.x, splits))


@pytest.mark.parametrize("k", [16, 528, 2048, 2064, 4096, 8192, 8208])
def test_rowwise_quantize_fused_and_fallback(k):
    # K <= 8192 runs the one-pass rowwise kernel (4, 8 or 16 column segments
    # per lane); K = 8208 falls back to amax + cast.  Both equal the oracle.
    w = synth.random_case(50 + k, [256, 0, 128], k, "outliers")
    check_small(w, True, False, entry="quantize")


def test_rowwise_graphsafe_quantize_equals_host_split():
    w = synth.random_case(61, [128, 384, 0, 256], 1040, "rowscale")
    splits = list(map(int, w.splits))
    log("graph-safe rowwise quantize")
    x = to_device(w.x)
    host = to_numpy(run_host_split(x, splits, True, False, entry="quantize"))
    out = alloc(w.sum_m, w.k, len(splits), True, False)
    d_offs = torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.nvfp4_group_quantize_graphsafe(x, len(splits), d_offs, d_status, **tensors(out))
    torch.cuda.synchronize()
    assert int(d_status.item()) == 0
    assert_guards(out)
    assert_equal_outputs(to_numpy(out), host)
    assert_equal_outputs(host, oracle_ref(w, True, False), ["row_amax", "row_data", "row_scale"])


@pytest.mark.parametrize("k", [1040, 4096, 8192, 8208])
def test_rowwise_graphsafe_quantize_partial_routing(k):
    # nvfp4_group_quantize_graphsafe with no columnwise output runs the fused
    # rowwise pass (K <= 8192; K = 8208 falls back to amax + cast); buffers
    # hold 1024 rows, the routing covers 640: rows 640.. keep their bytes and
    # the routed rows equal the oracle
    cap = 1024
    splits = [256, 0, 384]
    tot = sum(splits)
    rng = np.random.default_rng(62 + k)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((cap, k)).astype(np.float32))
    log(f"graph-safe rowwise quantize, partial routing, k={k}")
    x = to_device(xb)
    gs, status = _graphsafe(x, 3, B.offsets_from_splits(splits), cap, rowwise=True, columnwise=False,
                            prefill=0x5A, entry="quantize")
    assert status == 0
    assert_guards(gs)
    g = to_numpy(gs)
    assert (g["row_amax"][tot:].view(np.uint32) == 0x5A5A5A5A).all()
    assert (g["row_data"][tot:] == 0x5A).all() and (g["row_scale"][tot:] == 0x5A).all()
    ref = O.group_quantize(xb[:tot], splits, True, False)
    assert first_mismatch(g["row_amax"][:tot], ref["row_amax"]) is None
    assert first_mismatch(g["row_data"][:tot], ref["row_data"]) is None
    assert first_mismatch(g["row_scale"][:tot], ref["row_scale"]) is None


def test_many_experts_and_one_expert():
    # 96 experts of mixed sizes (many empty), and a single expert
    rng = np.random.default_rng(62)
    splits = (rng.integers(0, 3, 96) * 128).tolist()
    splits[5] = 0
    check_small(synth.random_case(63, splits, 80, "normal"))
    check_small(synth.random_case(64, [1024], 272, "rowscale"))


def test_max_host_experts_mostly_empty():
    splits = [0] * 512
    splits[0], splits[200], splits[511] = 128, 256, 128
    check_small(synth.random_case(65, splits, 32, "normal"))


# Small inputs with a columnwise output: nvfp4_group_quantize runs them as one
# launch (one work-group per expert); the bytes must be the oracle's.
SMALL_ONE_LAUNCH = [
    ([128, 0, 256, 128], 256, "normal", 91),        # the tiny workload's shape (largest expert at the limit)
    ([4096], 16, "normal", 92),                     # k = 16: the most rows one expert may have
    ([0, 128, 0], 512, "outliers", 93),             # k at its limit
    ([128, 0, 128], 272, "rowscale", 94),           # ragged 512-column chunk
    ([1280, 512], 48, "student", 95),               # gradient-like values, long experts
    ([128, 128, 128], 16, "sparse", 96),            # all-zero blocks and rows
    # expert counts that are not multiples of 8 (an expert's work-groups
    # share an XCD; indexes past the last expert exit)
    ([128] * 9, 64, "normal", 99),
    ([128, 0] * 16 + [256], 32, "rowscale", 100),
    ([0] * 70 + [128] * 3, 128, "student", 101),
]


@pytest.mark.parametrize("splits,k,dist,seed", SMALL_ONE_LAUNCH)
def test_small_input_one_launch(splits, k, dist, seed):
    assert max(splits) * k <= B.SMALL_MAX_EXPERT_ELEMS and k <= B.SMALL_MAX_K
    check_small(synth.random_case(seed, splits, k, dist), entry="quantize")


def test_small_input_one_launch_columnwise_only():
    check_small(synth.random_case(97, [256, 0, 128], 96, "rowscale"), rowwise=False, columnwise=True,
                entry="quantize")


def test_small_input_graphsafe_one_launch_many_experts():
    # device routing with 4093 experts (near the limit, not a multiple of the
    # 8 XCDs) over a 128-row capacity: every row in expert 4000, all others
    # empty (column amax 0); one launch
    rng = np.random.default_rng(102)
    cap, k, E = 128, 512, 4093
    assert E <= B.MAX_EXPERTS_DEVICE
    xb = synth.f32_to_bf16_bits(rng.standard_normal((cap, k)).astype(np.float32))
    splits = [0] * E
    splits[4000] = 128
    assert cap * k <= B.SMALL_MAX_EXPERT_ELEMS
    log("graph-safe one launch, 4093 experts")
    gs, status = _graphsafe(to_device(xb), E, B.offsets_from_splits(splits), cap, prefill=0x5A, entry="quantize")
    assert status == 0
    assert_guards(gs)
    assert_equal_outputs(to_numpy(gs), oracle_ref(synth.Workload("many", xb, np.array(splits, np.int64))))


def test_small_input_graphsafe_one_launch():
    # buffers for 512 rows, routing covers 384: the one-launch graph-safe
    # path writes the oracle's bytes and leaves rows 384.. as they were
    rng = np.random.default_rng(98)
    cap, k = 512, 96
    xb = synth.f32_to_bf16_bits(rng.standard_normal((cap, k)).astype(np.float32))
    splits = [256, 0, 128]
    assert cap * k <= B.SMALL_MAX_EXPERT_ELEMS
    log("graph-safe one launch, partial routing")
    gs, status = _graphsafe(to_device(xb), 3, B.offsets_from_splits(splits), cap, prefill=0x5A, entry="quantize")
    assert status == 0
    assert_guards(gs)
    g = to_numpy(gs)
    tot = sum(splits)
    assert (g["row_amax"][tot:].view(np.uint32) == 0x5A5A5A5A).all()
    assert (g["row_data"][tot:] == 0x5A).all() and (g["row_scale"][tot:] == 0x5A).all()
    assert (g["col_data"][k * tot // 2:] == 0x5A).all() and (g["col_scale"][k * tot // 16:] == 0x5A).all()
    ref = oracle_ref(synth.Workload("partial", xb[:tot], np.array(splits, np.int64)))
    for key, n in (("row_amax", tot), ("row_data", tot), ("row_scale", tot), ("col_amax", None),
                   ("col_data", k * tot // 2), ("col_scale", k * tot // 16)):
        assert first_mismatch(g[key][:n] if n is not None else g[key], ref[key]) is None, key


def test_small_input_graphsafe_rejects_bad_routing():
    log("graph-safe one launch, bad device routing")
    x = torch.zeros((1024, 32), dtype=torch.int16, device="cuda:0")
    gs, status = _graphsafe(x, 3, [256, 128, 384], 1024, prefill=0x33, entry="quantize")
    assert status & B.NVFP4G_DEV_NONMONO
    assert_guards(gs)
    for key, g in to_numpy(gs).items():
        assert (g.view(np.uint8) == 0x33).all(), key


def test_binding_launches_on_torch_current_stream():
    # the binding passes the handle of torch's current stream (the null
    # stream by default, a side stream inside torch.cuda.stream(...))
    assert (B._stream(None).value or 0) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert (B._stream(None).value or 0) == side.cuda_stream != 0


def _sweep_cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    dists = ["normal", "outliers", "rowscale", "student", "sparse"]
    cases = []
    for i in range(n):
        # even cases fit the one-launch limit (<= 256 rows per expert, k <= 256)
        small = i % 2 == 0
        E = int(rng.integers(1, 13))
        units = rng.integers(0, 3 if small else 4, E)  # groups of 128 rows, empty experts included
        if units.sum() == 0:
            units[int(rng.integers(0, E))] = 1
        k = 16 * int(rng.integers(1, 17 if small else 66))  # 16 .. 256 / 16 .. 1040
        cases.append(([int(u) * 128 for u in units], k, dists[i % len(dists)], 300 + i))
    return cases


@pytest.mark.parametrize("splits,k,dist,seed", _sweep_cases())
@pytest.mark.parametrize("entry", ["two_calls", "quantize"])
def test_random_sweep(splits, k, dist, seed, entry):
    # seeded random shapes and value mixes through both host entries (the
    # quantize entry takes the one-launch path where the experts are small)
    check_small(synth.random_case(seed, splits, k, dist), entry=entry)
