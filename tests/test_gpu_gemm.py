"""GPU row-scaled grouped GEMM (MFMA) against the oracle's float64 GEMM.

Operands are cast by the oracle on the CPU (never by the HIP path), uploaded,
multiplied on the GPU, and compared with the oracle's product of the
dequantised operands.

Tolerance (derived from the arithmetic): every product of two decoded
elements value(code) * value(S) is exact in fp32, so the only roundings are
the fp32 accumulation of the L products and the three fp32 operations of the
epilogue (two line scales A / 2688 and two multiplies).  With u = 2^-24 and
at most 2u per accumulation step (allowing for a truncating accumulator),
    |gpu - exact| <= (2 L + 8) u * sum_t |pa_t pb_t| * (Aa / 2688) (Ab / 2688),
the last factor being the oracle's `bound` output.  On operands whose partial
sums stay exactly representable (all block scales 448, line scales 1) the GPU
result must equal the oracle exactly, which pins the operand layouts.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import GUARD, Guarded, log

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def oracle_rowwise(bits: np.ndarray):
    """Oracle rowwise cast of any number of rows (zero rows pad the call to a
    multiple of 128): (data, scale, amax)."""
    rows, k = bits.shape
    pad = (-rows) % 128
    x = np.concatenate([bits, np.zeros((pad, k), np.uint16)]) if pad else bits
    q = O.group_quantize(np.ascontiguousarray(x), [rows + pad], rowwise=True, columnwise=False)
    return q["row_data"][:rows], q["row_scale"][:rows], q["row_amax"][:rows]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def run_fwd(a, b, splits, n, k, graphsafe=False, m_capacity=None):
    E = len(splits)
    sum_m = sum(splits)
    rows = m_capacity if graphsafe else sum_m
    out = Guarded(4 * rows * n, torch.float32, (rows, n))
    ta = [dev(v) for v in a]
    if graphsafe and rows > sum_m:   # operand rows beyond the routed ones: arbitrary bytes
        pad = rows - sum_m
        ta = [torch.cat([ta[0], torch.full((pad, k // 2), 0x77, dtype=torch.uint8, device="cuda:0")]),
              torch.cat([ta[1], torch.full((pad, k // 16), 0x38, dtype=torch.uint8, device="cuda:0")]),
              torch.cat([ta[2], torch.ones(pad, device="cuda:0")])]
    tb = [dev(b[0].reshape(E, n, k // 2)), dev(b[1].reshape(E, n, k // 16)), dev(b[2])]
    if graphsafe:
        d_offs = torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32, device="cuda:0")
        d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        B.nvfp4_group_gemm_graphsafe(*ta, *tb, d_offs, out.t, d_status)
        torch.cuda.synchronize()
        assert int(d_status.item()) == 0
    else:
        B.nvfp4_group_gemm(*ta, *tb, splits, out.t)
        torch.cuda.synchronize()
    assert out.guards_intact()
    return out


def check_close(got, want, bound, L, what):
    err = np.abs(got.astype(np.float64) - want)
    lim = (2 * L + 8) * U * bound + 1e-30
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    log(f"{what}: max |err| / bound = {ratio:.3e} (limit {(2 * L + 8) * U:.3e})")
    bad = np.argwhere(err > lim)
    assert bad.size == 0, f"{what}: {len(bad)} outside the bound; first {bad[0]}: gpu {got[tuple(bad[0])]} " \
                          f"oracle {want[tuple(bad[0])]}"


def _weights(rng, E, n, k, dist="normal"):
    w = rng.standard_normal((E * n, k)).astype(np.float32)
    if dist == "rowscale":
        w *= np.exp(rng.standard_normal((E * n, 1))).astype(np.float32)
    return oracle_rowwise(synth.f32_to_bf16_bits(w))


@pytest.mark.parametrize("splits,n,k,dist,seed", [
    ([128, 256, 0, 128], 272, 256, "rowscale", 81),     # ragged n (one partial column tile), empty expert
    ([384, 128], 48, 128, "outliers", 82),              # n below one column tile
    ([128] * 6, 512, 128, "normal", 83),                # a single contraction step
    ([1024, 0, 512, 2560], 320, 2048, "rowscale", 84),  # several row-tile groups, long contraction
    ([256, 128], 96, 384, "normal", 85),                # 3 steps: the first scale block partial
    ([128, 384, 0], 160, 896, "outliers", 86),          # 7 steps: the second scale block partial
])
def test_fwd_matches_oracle(splits, n, k, dist, seed):
    w = synth.random_case(seed, splits, k, dist)
    log(f"gemm fwd {w.name} n={n}")
    a = oracle_rowwise(w.x)
    rng = np.random.default_rng(seed + 1000)
    b = _weights(rng, len(splits), n, k, "rowscale")
    want, bound = O.group_gemm(*a, b[0].reshape(len(splits), n, -1), b[1].reshape(len(splits), n, -1), b[2],
                               splits, n, k)
    out = run_fwd(a, b, splits, n, k)
    check_close(out.numpy(), want, bound, k, f"fwd {w.name}")


def _exact_operand(rng, rows, k):
    """Values g * 448 with g on the E2M1 grid and a +-6 in every 16-block:
    block scales 448, line scale 1, so the cast is exact and every partial
    sum of products is a small multiple of 448^2 / 4 (exact in fp32)."""
    g = GRID[rng.integers(0, 8, (rows, k))] * rng.choice([-1.0, 1.0], (rows, k))
    g[np.arange(rows)[:, None], 16 * np.arange(k // 16)[None, :] + rng.integers(0, 16, (rows, k // 16))] = 6.0
    return g * 448.0


def test_fwd_exact_on_exactly_representable_operands():
    rng = np.random.default_rng(85)
    splits, n, k = [256, 128, 0, 384], 288, 384
    E = len(splits)
    X = _exact_operand(rng, sum(splits), k)
    W = _exact_operand(rng, E * n, k)
    a = oracle_rowwise(synth.f32_to_bf16_bits(X.astype(np.float32)))
    b = _weights_from(W)
    want, _ = O.group_gemm(*a, b[0].reshape(E, n, -1), b[1].reshape(E, n, -1), b[2], splits, n, k)
    r0 = 0
    for e, m in enumerate(splits):   # the oracle itself is the plain product here
        assert (want[r0:r0 + m] == X[r0:r0 + m] @ W[e * n:(e + 1) * n].T).all()
        r0 += m
    got = run_fwd(a, b, splits, n, k).numpy()
    bad = np.argwhere(got.astype(np.float64) != want)
    assert bad.size == 0, f"{len(bad)} inexact; first {bad[0]}: gpu {got[tuple(bad[0])]} oracle {want[tuple(bad[0])]}"


def _weights_from(W):
    return oracle_rowwise(synth.f32_to_bf16_bits(W.astype(np.float32)))


def test_fwd_graphsafe_equals_host_split_and_skips_unrouted_rows():
    rng = np.random.default_rng(86)
    splits, n, k = [256, 0, 128], 96, 256
    w = synth.random_case(86, splits, k, "normal")
    a = oracle_rowwise(w.x)
    b = _weights(rng, len(splits), n, k)
    host = run_fwd(a, b, splits, n, k).numpy()
    m_capacity = sum(splits) + 256
    g = run_fwd(a, b, splits, n, k, graphsafe=True, m_capacity=m_capacity)
    gn = g.numpy()
    assert (gn[:sum(splits)].view(np.uint32) == host.view(np.uint32)).all()
    raw = g.buf.cpu().numpy()[GUARD + 4 * sum(splits) * n: GUARD + 4 * m_capacity * n]
    assert (raw == 0xA5).all(), "rows beyond the routed total were written"


@pytest.mark.parametrize("splits,n,k,seed", [
    ([128, 0, 256, 128], 272, 48, 87),
    ([640, 384], 128, 512, 88),
    ([2048, 128], 64, 256, 89),
])
def test_wgrad_matches_oracle(splits, n, k, seed):
    log(f"gemm wgrad splits={splits} n={n} k={k}")
    dy = synth.random_case(seed, splits, n, "student")
    x = synth.random_case(seed + 1, splits, k, "rowscale")
    qy = O.group_quantize(dy.x, splits)
    qx = O.group_quantize(x.x, splits)
    want, bound = O.group_gemm_wgrad(qy["col_data"], qy["col_scale"], qy["col_amax"],
                                     qx["col_data"], qx["col_scale"], qx["col_amax"], splits, n, k)
    E = len(splits)
    out = Guarded(4 * E * n * k, torch.float32, (E, n, k))
    out.t.fill_(np.nan)
    B.nvfp4_group_gemm_wgrad(dev(qy["col_data"]), dev(qy["col_scale"]), dev(qy["col_amax"]),
                             dev(qx["col_data"]), dev(qx["col_scale"]), dev(qx["col_amax"]), splits, n, k, out.t)
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.numpy()
    for e, m in enumerate(splits):
        if m == 0:
            assert (got[e] == 0).all() and not np.signbit(got[e]).any(), "an expert without rows must give +0"
        else:
            check_close(got[e], want[e], bound[e], m, f"wgrad expert {e} (M_e={m})")


def test_wgrad_exact_on_exactly_representable_operands():
    rng = np.random.default_rng(90)
    splits, n, k = [256, 128], 48, 80
    # every row block and column block holds a +-6*448 on the diagonal
    def both(rows, cols):
        g = GRID[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
        r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
        g[(r % 16) == (c % 16)] = 6.0
        return g * 448.0
    dY, X = both(sum(splits), n), both(sum(splits), k)
    qy = O.group_quantize(synth.f32_to_bf16_bits(dY.astype(np.float32)), splits)
    qx = O.group_quantize(synth.f32_to_bf16_bits(X.astype(np.float32)), splits)
    want, _ = O.group_gemm_wgrad(qy["col_data"], qy["col_scale"], qy["col_amax"],
                                 qx["col_data"], qx["col_scale"], qx["col_amax"], splits, n, k)
    out = torch.empty((len(splits), n, k), dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_gemm_wgrad(dev(qy["col_data"]), dev(qy["col_scale"]), dev(qy["col_amax"]),
                             dev(qx["col_data"]), dev(qx["col_scale"]), dev(qx["col_amax"]), splits, n, k, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    r0 = 0
    for e, m in enumerate(splits):
        assert (want[e] == dY[r0:r0 + m].T @ X[r0:r0 + m]).all()
        r0 += m
    assert (got == want).all(), f"{int((got != want).sum())} inexact outputs"


def test_fwd_random_operand_bytes():
    # every code byte and every finite E4M3 scale code, subnormal scales and
    # zero scales included, so each decode step is exercised on all inputs
    rng = np.random.default_rng(91)
    splits, n, k = [128, 256], 80, 512
    E, sum_m = len(splits), sum(splits)
    a = (rng.integers(0, 256, (sum_m, k // 2), dtype=np.uint8), rng.integers(0, 0x7F, (sum_m, k // 16), dtype=np.uint8),
         rng.uniform(0.5, 2.0, sum_m).astype(np.float32))
    b = (rng.integers(0, 256, (E * n, k // 2), dtype=np.uint8), rng.integers(0, 0x7F, (E * n, k // 16), dtype=np.uint8),
         rng.uniform(0.5, 2.0, E * n).astype(np.float32))
    want, bound = O.group_gemm(*a, b[0].reshape(E, n, -1), b[1].reshape(E, n, -1), b[2], splits, n, k)
    out = run_fwd(a, b, splits, n, k)
    check_close(out.numpy(), want, bound, k, "fwd random bytes")


def test_wgrad_graphsafe_equals_host_split_and_replays():
    # the graph-safe weight gradient equals the host-split one bit for bit, and
    # one hipGraph capture replays under new routing written to the offsets
    rng = np.random.default_rng(92)
    n, k, e_n, m_cap = 48, 160, 4, 1024
    yd = rng.integers(0, 256, m_cap * n // 2, dtype=np.uint8)
    ys = rng.integers(0x20, 0x50, m_cap * n // 16, dtype=np.uint8)
    xd = rng.integers(0, 256, m_cap * k // 2, dtype=np.uint8)
    xs = rng.integers(0x20, 0x50, m_cap * k // 16, dtype=np.uint8)
    ya = rng.uniform(0.5, 2.0, e_n * n).astype(np.float32)
    xa = rng.uniform(0.5, 2.0, e_n * k).astype(np.float32)
    ops = [dev(v) for v in (yd, ys, ya, xd, xs, xa)]
    d_offs = torch.zeros(e_n, dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    out = torch.zeros((e_n, n, k), dtype=torch.float32, device="cuda:0")
    routes = [[256, 0, 512, 256], [128, 384, 0, 128], [0, 0, 0, 1024], [256, 256, 256, 256]]
    d_offs.copy_(torch.tensor(B.offsets_from_splits(routes[0]), dtype=torch.int32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.nvfp4_group_gemm_wgrad_graphsafe(*ops, m_cap, e_n, d_offs, n, k, out, d_status)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.nvfp4_group_gemm_wgrad_graphsafe(*ops, m_cap, e_n, d_offs, n, k, out, d_status)
    torch.cuda.synchronize()
    for i, sp in enumerate(routes):
        total = sum(sp)
        d_offs.copy_(torch.tensor(B.offsets_from_splits(sp), dtype=torch.int32))
        out.fill_(np.nan)
        g.replay()
        ref = torch.empty((e_n, n, k), dtype=torch.float32, device="cuda:0")
        B.nvfp4_group_gemm_wgrad(ops[0][:total * n // 2], ops[1][:total * n // 16], ops[2],
                                 ops[3][:total * k // 2], ops[4][:total * k // 16], ops[5], sp, n, k, ref)
        torch.cuda.synchronize()
        assert int(d_status.item()) == 0
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {i}"
        log(f"wgrad replay {i}: routing {sp} byte-identical to the host-split call")


@pytest.mark.parametrize("offs,bits", [
    ([256, 128, 384], B.NVFP4G_DEV_NONMONO),
    ([256, 300, 384], B.NVFP4G_DEV_UNALIGNED),
    ([256, 384, 1280], B.NVFP4G_DEV_OVERFLOW),
])
def test_graphsafe_gemms_reject_bad_routing(offs, bits):
    # bad device routing: both graph-safe GEMMs set the status bits and write
    # no output element
    rng = np.random.default_rng(94)
    E, n, k, m_cap = 3, 48, 128, 1024
    u8 = lambda *s: dev(rng.integers(0, 256, s, dtype=np.uint8))
    sc = lambda *s: dev(rng.integers(0x20, 0x50, s, dtype=np.uint8))
    amax = lambda m: dev(rng.uniform(0.5, 2.0, m).astype(np.float32))
    d_offs = torch.tensor(offs, dtype=torch.int32, device="cuda:0")
    log(f"graph-safe GEMMs, bad routing {offs}")

    out = torch.full((m_cap, n), -7.0, dtype=torch.float32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.nvfp4_group_gemm_graphsafe(u8(m_cap, k // 2), sc(m_cap, k // 16), amax(m_cap),
                                 u8(E, n, k // 2), sc(E, n, k // 16), amax(E * n), d_offs, out, d_status)
    torch.cuda.synchronize()
    assert int(d_status.item()) & bits
    assert bool((out == -7.0).all())

    dw = torch.full((E, n, k), -7.0, dtype=torch.float32, device="cuda:0")
    d_status.zero_()
    B.nvfp4_group_gemm_wgrad_graphsafe(u8(m_cap * n // 2), sc(m_cap * n // 16), amax(E * n),
                                       u8(m_cap * k // 2), sc(m_cap * k // 16), amax(E * k),
                                       m_cap, E, d_offs, n, k, dw, d_status)
    torch.cuda.synchronize()
    assert int(d_status.item()) & bits
    assert bool((dw == -7.0).all())
