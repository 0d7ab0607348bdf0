"""GPU dequantisation of row-scaled NVFP4 against the oracle's decode.

The kernel and the oracle use the same op order, x^ = (value(code) *
value(S)) * (A / 2688), so the fp32 results are compared bit for bit (a
stricter form of the max-abs-error <= 1e-6 cross-check).
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import Guarded, first_mismatch, log, run_host_split, to_device, to_numpy

pytestmark = pytest.mark.gpu


def oracle_columnwise_lines(q, splits, k):
    """Oracle decode of the transposed output, in its own layout."""
    out = np.empty(q["col_data"].size * 2, np.float32)
    r0 = 0
    for e, m in enumerate(splits):
        for c in range(k if m else 0):
            base = k * r0 + c * m
            out[base: base + m] = O.decode_line(q["col_data"][base // 2: (base + m) // 2],
                                                q["col_scale"][base // 16: (base + m) // 16], m,
                                                q["col_amax"][e * k + c])
        r0 += m
    return out


@pytest.mark.parametrize("splits,k,dist,seed", [
    ([128, 0, 256, 128], 272, "rowscale", 71),
    ([384, 128], 64, "outliers", 72),
    ([128, 128], 48, "sparse", 73),
])
def test_dequant_matches_oracle_decode(splits, k, dist, seed):
    w = synth.random_case(seed, splits, k, dist)
    log(f"dequant {w.name} k={k}")
    x = to_device(w.x)
    g = to_numpy(run_host_split(x, splits))
    t = {key: torch.from_numpy(np.ascontiguousarray(v)).cuda() for key, v in g.items()}
    out_r = Guarded(4 * w.sum_m * k, torch.float32, (w.sum_m, k))
    B.nvfp4_group_dequant_rowwise(t["row_data"], t["row_scale"], t["row_amax"], out_r.t)
    out_c = Guarded(4 * w.sum_m * k, torch.float32)
    B.nvfp4_group_dequant_columnwise(t["col_data"], t["col_scale"], t["col_amax"], splits, k, out_c.t)
    torch.cuda.synchronize()
    assert out_r.guards_intact() and out_c.guards_intact()
    ref_r = O.decode_rowwise(g["row_data"], g["row_scale"], g["row_amax"])
    assert first_mismatch(out_r.numpy(), ref_r) is None
    ref_c = oracle_columnwise_lines(g, splits, k)
    assert first_mismatch(out_c.numpy(), ref_c) is None


def test_dequant_closed_form_reproduces_input():
    rng = np.random.default_rng(74)
    M, K = 256, 96
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    gv = grid[rng.integers(0, 8, (M, K))] * rng.choice([-1.0, 1.0], (M, K))
    r, c = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    diag = (r % 16) == (c % 16)
    gv[diag] = 6.0 * rng.choice([-1.0, 1.0], int(diag.sum()))
    xf = (gv * 448.0 * 2.0 ** 3).astype(np.float32)
    splits = [128, 128]
    log("dequant closed form")
    x = to_device(synth.f32_to_bf16_bits(xf))
    g = to_numpy(run_host_split(x, splits))
    t = {key: torch.from_numpy(np.ascontiguousarray(v)).cuda() for key, v in g.items()}
    out_r = torch.empty((M, K), dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_dequant_rowwise(t["row_data"], t["row_scale"], t["row_amax"], out_r)
    out_c = torch.empty(M * K, dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_dequant_columnwise(t["col_data"], t["col_scale"], t["col_amax"], splits, K, out_c)
    torch.cuda.synchronize()
    assert (out_r.cpu().numpy().view(np.uint32) == xf.view(np.uint32)).all()
    xt = np.concatenate([np.ascontiguousarray(xf[0:128].T).reshape(-1), np.ascontiguousarray(xf[128:].T).reshape(-1)])
    assert (out_c.cpu().numpy().view(np.uint32) == xt.view(np.uint32)).all()


def test_dequant_columnwise_graphsafe_equals_host():
    w = synth.random_case(75, [256, 0, 384], 80, "rowscale")
    splits = list(map(int, w.splits))
    log("dequant graph-safe")
    x = to_device(w.x)
    g = to_numpy(run_host_split(x, splits))
    t = {key: torch.from_numpy(np.ascontiguousarray(v)).cuda() for key, v in g.items()}
    a = torch.empty(w.sum_m * w.k, dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_dequant_columnwise(t["col_data"], t["col_scale"], t["col_amax"], splits, w.k, a)
    b = torch.full((w.sum_m * w.k,), -7.0, dtype=torch.float32, device="cuda:0")
    d_offs = torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.nvfp4_group_dequant_columnwise_graphsafe(t["col_data"], t["col_scale"], t["col_amax"], w.sum_m, w.k,
                                               len(splits), d_offs, b, d_status)
    torch.cuda.synchronize()
    assert int(d_status.item()) == 0
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("rows,k", [(37, 48), (1, 16), (129, 2064), (300, 272)])
def test_dequant_rowwise_ragged_row_counts(rows, k):
    # row counts that leave a partial last 1024-element chunk (or a single block)
    w = synth.random_case(76 + rows, [((rows + 127) // 128) * 128], k, "outliers")
    log(f"dequant rowwise rows={rows} k={k}")
    g = to_numpy(run_host_split(to_device(w.x), list(map(int, w.splits)), True, False))
    rd, rs, ra = (np.ascontiguousarray(g[key][:rows]) for key in ("row_data", "row_scale", "row_amax"))
    out = Guarded(4 * rows * k, torch.float32, (rows, k))
    B.nvfp4_group_dequant_rowwise(*(torch.from_numpy(v).cuda() for v in (rd, rs, ra)), out.t)
    torch.cuda.synchronize()
    assert out.guards_intact()
    assert first_mismatch(out.numpy(), O.decode_rowwise(rd, rs, ra)) is None


def test_dequant_columnwise_many_small_experts_and_partial_routing():
    # 20 experts of 128 rows at K=16: every expert spans two 1024-element
    # chunks; the graph-safe call with capacity beyond the routed rows leaves
    # the tail of the output untouched
    splits = [128] * 20
    k = 16
    w = synth.random_case(77, splits, k, "rowscale")
    log("dequant columnwise, 20 experts")
    g = to_numpy(run_host_split(to_device(w.x), splits))
    t = {key: torch.from_numpy(np.ascontiguousarray(v)).cuda() for key, v in g.items()}
    out = Guarded(4 * w.sum_m * k, torch.float32)
    B.nvfp4_group_dequant_columnwise(t["col_data"], t["col_scale"], t["col_amax"], splits, k, out.t)
    torch.cuda.synchronize()
    assert out.guards_intact()
    assert first_mismatch(out.numpy(), oracle_columnwise_lines(g, splits, k)) is None
    part = splits[:13]
    cap = w.sum_m
    b = torch.full((cap * k,), -7.0, dtype=torch.float32, device="cuda:0")
    d_offs = torch.tensor(B.offsets_from_splits(part), dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.nvfp4_group_dequant_columnwise_graphsafe(t["col_data"], t["col_scale"], t["col_amax"], cap, k, len(part),
                                               d_offs, b, d_status)
    torch.cuda.synchronize()
    assert int(d_status.item()) == 0
    n = k * sum(part)
    got = b.cpu().numpy()
    assert first_mismatch(got[:n], out.numpy()[:n]) is None
    assert (got[n:] == -7.0).all()


@pytest.mark.parametrize("offs,bits", [
    ([256, 128, 384], B.NVFP4G_DEV_NONMONO),
    ([256, 300, 384], B.NVFP4G_DEV_UNALIGNED),
    ([256, 384, 1280], B.NVFP4G_DEV_OVERFLOW),
])
def test_dequant_columnwise_graphsafe_rejects_bad_routing(offs, bits):
    # bad device routing: the status bits are set and no output element is written
    rng = np.random.default_rng(76)
    cap, k = 1024, 64
    col_data = torch.from_numpy(rng.integers(0, 256, cap * k // 2, dtype=np.uint8)).cuda()
    col_scale = torch.from_numpy(rng.integers(0x20, 0x50, cap * k // 16, dtype=np.uint8)).cuda()
    col_amax = torch.ones(3 * k, dtype=torch.float32, device="cuda:0")
    out = torch.full((cap * k,), -7.0, dtype=torch.float32, device="cuda:0")
    d_offs = torch.tensor(offs, dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    log(f"dequant graph-safe bad routing {offs}")
    B.nvfp4_group_dequant_columnwise_graphsafe(col_data, col_scale, col_amax, cap, k, 3, d_offs, out, d_status)
    torch.cuda.synchronize()
    assert int(d_status.item()) & bits
    assert bool((out == -7.0).all())
