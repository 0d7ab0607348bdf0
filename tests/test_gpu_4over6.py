"""Parity of the four-over-six grouped cast (HIP, through the C ABI) with the
CPU oracle's four-over-six cast, element by element and bit-exact: small and
ragged shapes for every error mode and several scale bounds, each direction
alone, the graph-safe form under partial routing and under graph replay with
changed routing, the two full-size expert workloads on every byte, empty
inputs, and the ABI's size limits (2^24 rows, K = 2^22) on sampled lines.

The amax comes from the library's grouped amax (checked equal to the
oracle's); the four-over-six cast consumes it."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O
from oracle import parallel as OP

from gpu_helpers import alloc, assert_equal_outputs, assert_guards, log, tensors, to_device, to_numpy

pytestmark = pytest.mark.gpu

KNOBS = [(256, B.ERR_MSE), (448, B.ERR_MAE), (100, B.ERR_MSE), (1, B.ERR_MAE), (448, B.ERR_MSE), (37, B.ERR_MAE)]


def run_4o6(x_dev, splits, bound, mode, rowwise=True, columnwise=True):
    m, k = x_dev.shape
    out = alloc(m, k, len(splits), rowwise, columnwise)
    t = tensors(out)
    B.nvfp4_group_amax(x_dev, splits, t["row_amax"], t["col_amax"])
    B.nvfp4_group_cast_4over6(x_dev, splits, **t, scale_bound=bound, err_mode=mode)
    torch.cuda.synchronize()
    return out


def check(w, bound, mode, rowwise=True, columnwise=True):
    splits = list(map(int, w.splits))
    log(f"4over6 {w.name} m={w.sum_m} k={w.k} splits={splits} bound={bound} mode={mode} "
        f"row={rowwise} col={columnwise}")
    out = run_4o6(to_device(w.x), splits, bound, mode, rowwise, columnwise)
    assert_guards(out)
    gpu = to_numpy(out)
    ref = O.group_quantize_4o6(w.x, splits, bound, mode, rowwise, columnwise)
    assert_equal_outputs(gpu, ref)
    return gpu, ref


SMALL = [
    ([128, 0, 256, 128], 272, "normal", 31),       # 272 = 256 + 16: ragged column chunk
    ([384, 128], 48, "outliers", 32),
    ([256, 256, 0, 0, 512], 784, "outliers", 33),  # 784 = 3*256 + 16
    ([128, 128, 128], 16, "sparse", 34),           # all-zero blocks and rows
    ([640, 128], 2064, "rowscale", 35),
    ([0, 256, 128, 0], 512, "student", 36),        # gradient-like small values
    ([128] * 9, 96, "normal", 37),
]


@pytest.mark.parametrize("knob", range(len(KNOBS)))
def test_tiny_config_every_knob(knob):
    bound, mode = KNOBS[knob]
    check(synth.tiny(), bound, mode)


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_ragged_cases(case):
    splits, k, dist, seed = SMALL[case]
    w = synth.random_case(seed, splits, k, dist)
    for bound, mode in (KNOBS[case % len(KNOBS)], KNOBS[(case + 3) % len(KNOBS)]):
        check(w, bound, mode)


@pytest.mark.parametrize("rowwise,columnwise", [(True, False), (False, True)])
def test_one_direction(rowwise, columnwise):
    w = synth.random_case(41, [256, 128, 0, 384], 1040, "normal")
    check(w, 256, B.ERR_MSE, rowwise, columnwise)


@pytest.mark.parametrize("bound,mode", [(1, B.ERR_MSE), (256, B.ERR_MAE), (448, B.ERR_MSE)])
def test_tiny_and_huge_lines(bound, mode):
    """Lines whose scale steps leave the fast quotients' ranges: bf16
    subnormals and tiny normals (line scale below 2^-112, d and 1/d beyond
    the normal range), huge rows (d at or above 2^126, up to overflow, so
    m = 0 and the errors overflow), and ordinary rows in between; the
    columns mix all of them."""
    rng = np.random.default_rng(51)
    M, K = 384, 80
    v = rng.standard_normal((M, K)).astype(np.float32)
    row_exp = rng.integers(-133, -95, (M, 1)).astype(np.float32)
    v = v * np.exp2(row_exp)
    v[::7] *= np.float32(2.0 ** 60)           # ordinary rows
    v[3::11] = (rng.standard_normal((len(range(3, M, 11)), K)) * 2.0 ** 120).astype(np.float32)  # huge rows
    w = synth.Workload("tiny_huge", synth.f32_to_bf16_bits(v), np.array([128, 256], np.int64))
    check(w, bound, mode)


def test_huge_outlier_next_to_tiny_values():
    """A huge value in each line with tiny values around it: most blocks get
    subnormal or zero scales for both candidates."""
    rng = np.random.default_rng(52)
    M, K = 256, 64
    v = (rng.standard_normal((M, K)) * 1e-6).astype(np.float32)
    v[np.arange(M), rng.integers(0, K, M)] = np.float32(3e4)
    w = synth.Workload("extremes", synth.f32_to_bf16_bits(v), np.array([256], np.int64))
    for bound, mode in ((256, B.ERR_MSE), (7, B.ERR_MAE)):
        check(w, bound, mode)


def test_both_candidates_are_taken():
    """The parity above is only meaningful if blocks pick both encodings: on
    the normal workload about half of the blocks keep k = 4; with bound 448
    the k = 6 candidate is the plain cast's, so the blocks whose scale byte
    differs from the plain cast are exactly the k = 4 picks."""
    w = synth.random_case(42, [256, 256], 512, "normal")
    gpu, _ = check(w, 448, B.ERR_MSE)
    plain = O.group_quantize(w.x, list(map(int, w.splits)))
    frac_row = float((gpu["row_scale"] != plain["row_scale"]).mean())
    frac_col = float((gpu["col_scale"] != plain["col_scale"]).mean())
    log(f"blocks taking k = 4: rowwise {frac_row:.3f}, columnwise {frac_col:.3f}")
    assert 0.1 < frac_row < 0.9 and 0.1 < frac_col < 0.9


def test_graphsafe_partial_routing_leaves_the_tail_untouched():
    """Capacity 1024 rows, routed 640: the routed rows equal the oracle's
    four-over-six cast of those rows, and nothing at or beyond the routed
    total is written."""
    k, cap, splits = 1040, 1024, [256, 0, 384]
    w = synth.random_case(43, [cap], k, "normal")
    x_dev = to_device(w.x)
    routed = sum(splits)
    offs = torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    out = alloc(cap, k, len(splits), True, True)
    for g in out.values():
        g.t.view(torch.uint8).fill_(0x5A)
    t = tensors(out)
    log(f"4over6 graphsafe partial routing cap={cap} routed={routed} k={k}")
    B.nvfp4_group_amax_graphsafe(x_dev, len(splits), offs, status, t["row_amax"], t["col_amax"])
    B.nvfp4_group_cast_4over6_graphsafe(x_dev, len(splits), offs, status, **t, scale_bound=256,
                                        err_mode=B.ERR_MSE)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_guards(out)
    gpu = {key: g.numpy() for key, g in out.items()}
    ref = O.group_quantize_4o6(w.x[:routed], splits, 256, B.ERR_MSE)
    assert np.array_equal(gpu["row_data"][:routed], ref["row_data"])
    assert np.array_equal(gpu["row_scale"][:routed], ref["row_scale"])
    assert np.array_equal(gpu["col_data"][:k * routed // 2], ref["col_data"])
    assert np.array_equal(gpu["col_scale"][:k * routed // 16], ref["col_scale"])
    assert (gpu["row_data"][routed:] == 0x5A).all() and (gpu["row_scale"][routed:] == 0x5A).all()
    assert (gpu["col_data"][k * routed // 2:] == 0x5A).all()
    assert (gpu["col_scale"][k * routed // 16:] == 0x5A).all()


def test_graph_replay_changed_routing_equals_host_split():
    """One capture of the graph-safe amax + four-over-six cast, replayed
    under three routings: each replay is byte-identical to the host-split
    calls for that routing, and the first equals the oracle."""
    k, cap, E = 768, 2048, 4
    w = synth.random_case(44, [cap], k, "normal")
    x_dev = to_device(w.x)
    routings = [[512, 0, 1024, 512], [128, 1664, 128, 128], [0, 0, 0, 1920]]
    offs = torch.zeros(E, dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    bufs = B.alloc_outputs(cap, k, E)
    offs.copy_(torch.tensor(B.offsets_from_splits(routings[0]), dtype=torch.int32, device="cuda:0"))

    def step():
        B.nvfp4_group_amax_graphsafe(x_dev, E, offs, status, bufs["row_amax"], bufs["col_amax"])
        B.nvfp4_group_cast_4over6_graphsafe(x_dev, E, offs, status, **bufs, scale_bound=256, err_mode=B.ERR_MAE)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for n, sp in enumerate(routings):
        log(f"4over6 graph replay {n} routing {sp}")
        offs.copy_(torch.tensor(B.offsets_from_splits(sp), dtype=torch.int32, device="cuda:0"))
        for t in bufs.values():
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        routed = sum(sp)
        host = B.alloc_outputs(routed, k, E)
        B.nvfp4_group_amax(x_dev[:routed], sp, host["row_amax"], host["col_amax"])
        B.nvfp4_group_cast_4over6(x_dev[:routed], sp, **host, scale_bound=256, err_mode=B.ERR_MAE)
        torch.cuda.synchronize()
        assert torch.equal(bufs["row_amax"][:routed], host["row_amax"])
        assert torch.equal(bufs["col_amax"], host["col_amax"])
        assert torch.equal(bufs["row_data"][:routed], host["row_data"])
        assert torch.equal(bufs["row_scale"][:routed], host["row_scale"])
        assert torch.equal(bufs["col_data"][:k * routed // 2], host["col_data"])
        assert torch.equal(bufs["col_scale"][:k * routed // 16], host["col_scale"])
        if n == 0:
            ref = O.group_quantize_4o6(w.x[:routed], sp, 256, B.ERR_MAE)
            assert np.array_equal(host["row_data"].cpu().numpy(), ref["row_data"])
            assert np.array_equal(host["col_data"].cpu().numpy(), ref["col_data"])
            assert np.array_equal(host["row_scale"].cpu().numpy(), ref["row_scale"])
            assert np.array_equal(host["col_scale"].cpu().numpy(), ref["col_scale"])


FULL = [("deepseek_share", 256, B.ERR_MSE), ("down_proj", 448, B.ERR_MAE)]


@pytest.mark.parametrize("name,bound,mode", FULL)
def test_full_size_every_byte(name, bound, mode):
    """The expert-share (65536 x 7168, 32 experts) and down-projection
    (131072 x 2048, 64 experts) workloads, both directions: every amax, data
    byte and scale byte against the oracle (run as independent row-range and
    column-range calls on a thread pool)."""
    w = getattr(synth, name)()
    splits = list(map(int, w.splits))
    log(f"4over6 full size {name} bound={bound} mode={mode}: GPU")
    x_dev = to_device(w.x)
    bufs = B.alloc_outputs(w.sum_m, w.k, len(splits))
    B.nvfp4_group_amax(x_dev, splits, bufs["row_amax"], bufs["col_amax"])
    B.nvfp4_group_cast_4over6(x_dev, splits, **bufs, scale_bound=bound, err_mode=mode)
    torch.cuda.synchronize()
    gpu = {key: t.cpu().numpy() for key, t in bufs.items()}
    del x_dev, bufs
    log(f"4over6 full size {name}: oracle")
    ref = OP.group_quantize(w.x, splits, True, True, four_over_six=(bound, mode))
    log(f"4over6 full size {name}: compare")
    for key in ("row_amax", "col_amax"):
        assert np.array_equal(gpu[key].view(np.uint32), ref[key].view(np.uint32)), key
    for key in ("row_data", "row_scale", "col_data", "col_scale"):
        a, b = gpu[key].reshape(-1), ref[key].reshape(-1)
        bad = np.count_nonzero(a != b)
        assert bad == 0, f"{key}: {bad} mismatching bytes"


def test_empty_inputs():
    """No routed rows: the host-split call with all-empty experts and the
    graph-safe call with zero offsets succeed and write nothing."""
    k = 64
    x = torch.zeros((0, k), dtype=torch.int16, device="cuda:0")
    out = B.alloc_outputs(0, k, 3)
    log("4over6 empty host-split call")
    B.nvfp4_group_amax(x, [0, 0, 0], out["row_amax"], out["col_amax"])
    B.nvfp4_group_cast_4over6(x, [0, 0, 0], **out)
    cap = 256
    xc = torch.zeros((cap, k), dtype=torch.int16, device="cuda:0")
    o = alloc(cap, k, 3, True, True)
    for g in o.values():
        g.t.view(torch.uint8).fill_(0x5A)
    t = tensors(o)
    t["row_amax"].zero_()
    t["col_amax"].zero_()
    offs = torch.zeros(3, dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    log("4over6 empty graph-safe call")
    B.nvfp4_group_cast_4over6_graphsafe(xc, 3, offs, status, **t)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_guards(o)
    for key in ("row_data", "row_scale", "col_data", "col_scale"):
        assert (o[key].numpy() == 0x5A).all(), key


def _line_ref(L, A, bound, mode):
    d, s, _ = O.encode_line_4o6(synth.bf16_bits_to_f32(L), float(A), bound, mode)
    return d, s


def test_row_limit_2_to_24_rows():
    """2^24 rows at K = 16 (two experts, one of 2^24 - 2^17 rows): the
    largest row offsets.  Sampled rows (both ends of each expert and random
    ones) and whole column lines against the oracle's line encoder."""
    bound, mode = 256, B.ERR_MSE
    log("4over6 row limit: generating 2^24 x 16")
    w = synth.max_rows()
    splits = list(map(int, w.splits))
    x = to_device(w.x)
    out = B.alloc_outputs(w.sum_m, w.k, len(splits))
    B.nvfp4_group_amax(x, splits, out["row_amax"], out["col_amax"])
    B.nvfp4_group_cast_4over6(x, splits, **out, scale_bound=bound, err_mode=mode)
    torch.cuda.synchronize()
    res = {key: t.cpu().numpy() for key, t in out.items()}
    del x, out
    rng = np.random.default_rng(61)
    offs = np.concatenate([[0], np.cumsum(splits)]).astype(np.int64)
    rows = set(rng.integers(0, w.sum_m, 2000).tolist())
    for e in range(len(splits)):
        rows |= {int(offs[e]), int(offs[e]) + 1, int(offs[e + 1]) - 1}
    log(f"4over6 row limit: {len(rows)} rows vs oracle")
    for r in sorted(rows):
        d, s = _line_ref(w.x[r], res["row_amax"][r], bound, mode)
        assert np.array_equal(res["row_data"][r], d) and np.array_equal(res["row_scale"][r], s), f"row {r}"
    k = w.k
    for e in range(len(splits)):
        r0, m = int(offs[e]), splits[e]
        for c in (0, 7, 15):
            log(f"4over6 row limit: expert {e} column {c} ({m} rows) vs oracle")
            d, s = _line_ref(np.ascontiguousarray(w.x[r0:r0 + m, c]), res["col_amax"][e * k + c], bound, mode)
            d0, s0 = k * r0 // 2 + c * (m // 2), k * r0 // 16 + c * (m // 16)
            assert np.array_equal(res["col_data"][d0:d0 + m // 2], d), f"col_data expert {e} column {c}"
            assert np.array_equal(res["col_scale"][s0:s0 + m // 16], s), f"col_scale expert {e} column {c}"


def test_column_limit_k_2_to_22():
    """K = 2^22 (one expert of 128 rows): the largest column offsets.
    Sampled rows and 20000 sampled column lines against the oracle's line
    encoder, and the graph-safe call byte-identical to the host-split one."""
    bound, mode = 448, B.ERR_MAE
    log("4over6 column limit: generating 128 x 2^22")
    w = synth.max_k()
    splits = list(map(int, w.splits))
    x = to_device(w.x)
    out = B.alloc_outputs(w.sum_m, w.k, 1)
    B.nvfp4_group_amax(x, splits, out["row_amax"], out["col_amax"])
    B.nvfp4_group_cast_4over6(x, splits, **out, scale_bound=bound, err_mode=mode)
    g = B.alloc_outputs(w.sum_m, w.k, 1)
    g["row_amax"].copy_(out["row_amax"])
    g["col_amax"].copy_(out["col_amax"])
    offs = torch.tensor([w.sum_m], dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.nvfp4_group_cast_4over6_graphsafe(x, 1, offs, status, **g, scale_bound=bound, err_mode=mode)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for key in out:
        assert torch.equal(out[key], g[key]), key
    res = {key: t.cpu().numpy() for key, t in out.items()}
    del x, out, g
    k, m = w.k, w.sum_m
    for r in (0, 1, 63, 126, 127):
        log(f"4over6 column limit: row {r} vs oracle")
        d, s = _line_ref(w.x[r], res["row_amax"][r], bound, mode)
        assert np.array_equal(res["row_data"][r], d) and np.array_equal(res["row_scale"][r], s), f"row {r}"
    rng = np.random.default_rng(62)
    cols = np.unique(np.concatenate([rng.integers(0, k, 20000), [0, 1, k - 2, k - 1]]))
    log(f"4over6 column limit: {cols.size} column lines vs oracle")
    for c in cols.tolist():
        d, s = _line_ref(np.ascontiguousarray(w.x[:, c]), res["col_amax"][c], bound, mode)
        assert np.array_equal(res["col_data"][c * (m // 2):(c + 1) * (m // 2)], d), f"col_data column {c}"
        assert np.array_equal(res["col_scale"][c * (m // 16):(c + 1) * (m // 16)], s), f"col_scale column {c}"


@pytest.mark.parametrize("offs,bits", [
    ([256, 128, 384], B.NVFP4G_DEV_NONMONO),
    ([256, 300, 384], B.NVFP4G_DEV_UNALIGNED),
    ([256, 384, 1280], B.NVFP4G_DEV_OVERFLOW),
])
def test_graphsafe_rejects_bad_device_routing(offs, bits):
    """Invalid device routing: the status bit is set and no output byte is
    written (the amax buffers hold a prefill the cast would otherwise read)."""
    log(f"4over6 bad device routing {offs}")
    cap, k = 1024, 32
    x = torch.zeros((cap, k), dtype=torch.int16, device="cuda:0")
    o = alloc(cap, k, 3, True, True)
    for g in o.values():
        g.t.view(torch.uint8).fill_(0x33)
    d_offs = torch.tensor(offs, dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.nvfp4_group_cast_4over6_graphsafe(x, 3, d_offs, status, **tensors(o), scale_bound=256, err_mode=B.ERR_MSE)
    torch.cuda.synchronize()
    assert int(status.item()) & bits
    assert_guards(o)
    for key, g in o.items():
        assert (g.numpy().view(np.uint8) == 0x33).all(), key
