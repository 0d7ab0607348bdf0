"""Parity of the grouped MXFP4 cast (HIP path, through the C ABI) with the
CPU oracle, bit-exact on every data and scale byte.

Small seeded cases span several 128 x 256 tiles, ragged column chunks
(K a multiple of 32 but not of 256), zero-row experts, signed zeros,
subnormal and near-maximal bf16 values; the expert-share workload
(32 experts, K=7168, sum_M=65536) is compared element by element at full
size.  The graph-safe entry is checked against the host-split one, on
partial and invalid routing, and under hipGraph replay with new routing.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import Guarded, assert_guards, first_mismatch, log, to_device

pytestmark = pytest.mark.gpu

KEYS = ("row_data", "row_scale", "col_data", "col_scale")


def alloc_mx(m_rows, k, rowwise=True, columnwise=True, prefill=None):
    out = {}
    if rowwise:
        out["row_data"] = Guarded(m_rows * k // 2, torch.uint8, (m_rows, k // 2))
        out["row_scale"] = Guarded(m_rows * k // 32, torch.uint8, (m_rows, k // 32))
    if columnwise:
        out["col_data"] = Guarded(m_rows * k // 2)
        out["col_scale"] = Guarded(m_rows * k // 32)
    if prefill is not None:
        for g in out.values():
            g.t.fill_(prefill)
    return out


def tensors(out):
    return {key: (out[key].t if key in out else None) for key in KEYS}


def numpy_out(out):
    return {key: g.numpy() for key, g in out.items()}


def run_mx(x_dev, splits, rowwise=True, columnwise=True):
    out = alloc_mx(x_dev.shape[0], x_dev.shape[1], rowwise, columnwise)
    B.mxfp4_group_cast(x_dev, splits, **tensors(out))
    torch.cuda.synchronize()
    assert_guards(out)
    return out


def oracle_mx(x_bits, splits, rowwise=True, columnwise=True):
    rd, rs, cd, cs = O.mxfp4_group_cast(x_bits, splits, rowwise, columnwise)
    return {key: v for key, v in zip(KEYS, (rd, rs, cd, cs)) if v is not None}


def assert_same(gpu, ref):
    assert set(gpu) == set(ref)
    for key in ref:
        msg = first_mismatch(gpu[key], ref[key])
        assert msg is None, f"{key}: {msg}"


def check(x_bits, splits, rowwise=True, columnwise=True, name=""):
    splits = [int(v) for v in splits]
    log(f"mxfp4 {name} m={x_bits.shape[0]} k={x_bits.shape[1]} splits={splits} row={rowwise} col={columnwise}")
    gpu = numpy_out(run_mx(to_device(x_bits), splits, rowwise, columnwise))
    assert_same(gpu, oracle_mx(x_bits, splits, rowwise, columnwise))
    return gpu


SMALL = [
    ([128, 0, 256, 128], 288, "normal", 71),       # 288 = 256 + 32: ragged column chunk
    ([384, 128], 32, "outliers", 72),
    ([256, 256, 0, 0, 512], 800, "outliers", 73),  # 800 = 3*256 + 32
    ([128, 128, 128], 64, "sparse", 74),           # all-zero blocks
    ([640, 128], 2080, "rowscale", 75),
    ([0, 256, 128, 0], 512, "student", 76),
    ([128] * 9, 96, "normal", 77),
]


@pytest.mark.parametrize("splits,k,dist,seed", SMALL)
def test_small_cases(splits, k, dist, seed):
    w = synth.random_case(seed, splits, k, dist)
    check(w.x, w.splits, name=w.name)


@pytest.mark.parametrize("rowwise,columnwise", [(True, False), (False, True)])
def test_single_direction(rowwise, columnwise):
    w = synth.random_case(78, [256, 128, 0, 384], 352, "rowscale")
    check(w.x, w.splits, rowwise, columnwise, name=w.name)


def _extreme_bits(rng, shape):
    """bf16 bit patterns mixing every exponent class: signed zeros,
    subnormals, the smallest normals, ordinary values and values up to the
    largest finite bf16 (exponent field 254), with random signs."""
    n = int(np.prod(shape))
    kind = rng.integers(0, 6, n)
    exp = np.where(kind == 0, 0,                                      # zero / subnormal
          np.where(kind == 1, rng.integers(1, 4, n),                  # smallest normals
          np.where(kind == 2, rng.integers(100, 140, n),              # ordinary
          np.where(kind == 3, rng.integers(240, 255, n),              # huge
                   rng.integers(1, 255, n)))))                        # anything finite
    man = rng.integers(0, 128, n)
    man = np.where((kind == 0) & (rng.random(n) < 0.3), 0, man)       # exact zeros
    sign = rng.integers(0, 2, n)
    bits = (sign << 15) | (exp << 7) | man
    return bits.astype(np.uint16).reshape(shape)


def test_extreme_exponents():
    rng = np.random.default_rng(79)
    x = _extreme_bits(rng, (512, 320))
    check(x, [128, 256, 128], name="extreme exponents")


def test_block_classes():
    # rows / columns whose 32-blocks are: all zero (byte 0), negative zeros
    # only (codes 8), one subnormal (byte 0), a tiny value beside a huge one
    # (product underflows to a signed zero), exactly powers of two (the
    # block amax on an exponent boundary) and the bf16 maximum (byte 252)
    rows, k = 256, 256
    f = np.zeros((rows, k), np.float32)
    f[1] = -0.0
    f[2, 5] = 2.0 ** -133
    f[3, :] = 1e-38
    f[3, 7] = 3.0e38
    f[4] = (2.0 ** np.arange(-128, 128, dtype=np.float64)).astype(np.float32)
    f[5] = np.float32(3.3895314e38) * np.where(np.arange(k) % 2, 1, -1)
    f[6] = np.linspace(-6.0, 6.0, k, dtype=np.float32)            # ties of E2M1 at shared = 0
    f[7] = (np.arange(k) % 16 - 8).astype(np.float32) * 0.25       # exact multiples of 0.25
    f[8:] = np.random.default_rng(80).standard_normal((rows - 8, k)).astype(np.float32)
    x = synth.f32_to_bf16_bits(f)
    x[1] = 0x8000
    gpu = check(x, [128, 128], name="block classes")
    assert (gpu["row_scale"][0] == 0).all() and (gpu["row_data"][0] == 0).all()
    assert (gpu["row_data"][1] == 0x88).all()
    assert (gpu["row_scale"][5] == 252).all()


def test_empty_input_and_empty_experts():
    log("mxfp4 empty input")
    x = torch.zeros((0, 64), dtype=torch.int16, device="cuda:0")
    out = alloc_mx(0, 64)
    B.mxfp4_group_cast(x, [0, 0, 0], **tensors(out))
    torch.cuda.synchronize()
    assert_guards(out)
    w = synth.random_case(81, [0, 0, 384, 0], 128, "normal")
    check(w.x, w.splits, name="leading/trailing empty experts")


def test_deterministic():
    w = synth.random_case(82, [256, 512], 544, "student")
    x = to_device(w.x)
    a = numpy_out(run_mx(x, list(map(int, w.splits))))
    b = numpy_out(run_mx(x, list(map(int, w.splits))))
    assert_same(a, b)


# ----------------------------------------------------------- graph-safe path

def _graphsafe(x_dev, E, offs, m_cap, rowwise=True, columnwise=True, prefill=None):
    out = alloc_mx(m_cap, x_dev.shape[1], rowwise, columnwise, prefill)
    d_offs = torch.tensor(offs, dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.mxfp4_group_cast_graphsafe(x_dev, E, d_offs, d_status, **tensors(out))
    torch.cuda.synchronize()
    assert_guards(out)
    return numpy_out(out), int(d_status.item())


def test_graphsafe_matches_host_split_and_leaves_the_tail():
    rng = np.random.default_rng(83)
    cap, k = 1280, 416
    xb = synth.f32_to_bf16_bits(rng.standard_normal((cap, k)).astype(np.float32))
    splits = [384, 0, 128, 256]
    tot = sum(splits)
    log("mxfp4 graph-safe partial routing")
    x = to_device(xb)
    gs, status = _graphsafe(x, len(splits), B.offsets_from_splits(splits), cap, prefill=0x5A)
    assert status == 0
    assert (gs["row_data"][tot:] == 0x5A).all() and (gs["row_scale"][tot:] == 0x5A).all()
    assert (gs["col_data"][k * tot // 2:] == 0x5A).all() and (gs["col_scale"][k * tot // 32:] == 0x5A).all()
    ref = oracle_mx(xb[:tot], splits)
    got = {"row_data": gs["row_data"][:tot], "row_scale": gs["row_scale"][:tot],
           "col_data": gs["col_data"][:k * tot // 2], "col_scale": gs["col_scale"][:k * tot // 32]}
    assert_same(got, ref)
    host = numpy_out(run_mx(to_device(xb[:tot]), splits))
    assert_same(got, host)


@pytest.mark.parametrize("offs,bits", [
    ([256, 128, 384], B.NVFP4G_DEV_NONMONO),
    ([256, 300, 384], B.NVFP4G_DEV_UNALIGNED),
    ([256, 384, 1280], B.NVFP4G_DEV_OVERFLOW),
])
def test_graphsafe_rejects_bad_device_routing(offs, bits):
    log(f"mxfp4 bad device routing {offs}")
    x = torch.zeros((1024, 64), dtype=torch.int16, device="cuda:0")
    gs, status = _graphsafe(x, 3, offs, 1024, prefill=0x33)
    assert status & bits
    for key, g in gs.items():
        assert (g == 0x33).all(), key


def test_graph_capture_replays_under_new_routing():
    rng = np.random.default_rng(84)
    E, cap, k = 8, 2048, 480
    xb = synth.f32_to_bf16_bits((rng.standard_t(3.0, (cap, k)) * 1e-3).astype(np.float32))
    x = to_device(xb)
    out = alloc_mx(cap, k)
    t = tensors(out)
    d_offs = torch.zeros(E, dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def routing(i):
        units = np.random.default_rng(200 + i).multinomial(cap // 128, np.full(E, 1.0 / E))
        return [int(u) * 128 for u in units]

    log("mxfp4 graph capture")
    d_offs.copy_(torch.tensor(B.offsets_from_splits(routing(0)), dtype=torch.int32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.mxfp4_group_cast_graphsafe(x, E, d_offs, d_status, **t)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.mxfp4_group_cast_graphsafe(x, E, d_offs, d_status, **t)
    for i in range(5):
        splits = routing(i)
        log(f"mxfp4 replay {i} splits={splits}")
        d_offs.copy_(torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        got = numpy_out(out)
        host = numpy_out(run_mx(x, splits))
        assert_same(got, host)
        if i in (0, 4):
            assert_same(host, oracle_mx(xb, splits))
    assert int(d_status.item()) == 0
    assert_guards(out)


# ------------------------------------------------------------------ full size

def test_expert_share_full_size_elementwise():
    # 32 experts, K=7168, sum_M=65536 (Zipf-skewed splits): every byte of
    # both directions against the oracle
    w = synth.deepseek_share()
    splits = list(map(int, w.splits))
    log(f"mxfp4 {w.name} splits={splits}")
    gpu = numpy_out(run_mx(to_device(w.x), splits))
    log("mxfp4 oracle at full size")
    assert_same(gpu, oracle_mx(w.x, splits))
