"""The amax + cast at the size limits of the C ABI, where the kernels' 32-bit
buffer offsets are largest: 2^24 rows (K = 16, two experts, one of
2^24 - 2^17 rows) and K = 2^22 columns (128 rows).  Inputs are seeded
row-scaled normals (synth.max_rows, synth.max_k).  Checked against the oracle
line by line where it can afford it, and elsewhere by properties that hold at
any size: the row and column amax equal the maximum of |x| over the line
(exact, compared on bf16 bit patterns, which order non-negative values), the
graph-safe call equals the host-split one byte for byte, and the rowwise-only
request at K = 2^22 equals the rowwise half of the both-directions call.  The
MXFP4 cast (2^24 rows at K = 32, and K = 2^22) and the dequant (seeded
encoded bytes at both limits) are checked on sampled lines against the
oracle the same way.  The grouped GEMM is run at its limits (contraction
k = 2^22, n = 2^20, 2^22 rows per expert in the weight gradient) on operands
whose fp32 sums are exact (element values 0, +-0.5, +-1, unit scales), so its
outputs must equal the oracle's float64 dot products exactly.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _run(w, rowwise=True, columnwise=True):
    dev = torch.device("cuda:0")
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    out = B.alloc_outputs(w.sum_m, w.k, w.num_experts, rowwise, columnwise, device=dev)
    B.nvfp4_group_quantize(x, [int(v) for v in w.splits], **out)
    torch.cuda.synchronize()
    return x, out


def _abs_bits(x):
    return (x & np.uint16(0x7FFF)).astype(np.uint16)


def _amax_from_bits(b16):
    return (b16.astype(np.uint32) << 16).view(np.float32)


def _check_col_line(w, out, e, c):
    offs = np.concatenate([[0], np.cumsum(w.splits)]).astype(np.int64)
    r0, m, k = int(offs[e]), int(w.splits[e]), w.k
    A = O.col_amax(w.x, c, r0, m)
    assert out["col_amax"][e * k + c] == A, f"col_amax[{e}, {c}]"
    d, s = O.cast_col(w.x, c, r0, m, A)
    d0, s0 = k * r0 // 2 + c * (m // 2), k * r0 // 16 + c * (m // 16)
    assert np.array_equal(out["col_data"][d0:d0 + m // 2], d), f"col_data expert {e} column {c}"
    assert np.array_equal(out["col_scale"][s0:s0 + m // 16], s), f"col_scale expert {e} column {c}"


def _check_row(w, out, r):
    A = O.row_amax(w.x, r)
    assert out["row_amax"][r] == A, f"row_amax[{r}]"
    d, s = O.cast_row(w.x, r, A)
    assert np.array_equal(out["row_data"][r], d), f"row_data[{r}]"
    assert np.array_equal(out["row_scale"][r], s), f"row_scale[{r}]"


def test_row_limit_2_to_24_rows():
    log("generating 2^24 x 16")
    w = synth.max_rows()
    log(f"quantize {w.name}")
    x, dout = _run(w)
    out = {key: t.cpu().numpy() for key, t in dout.items()}
    # every row amax: the max of |x| over the row (exact)
    want = _amax_from_bits(_abs_bits(w.x).max(axis=1))
    assert np.array_equal(out["row_amax"].view(np.uint32), want.view(np.uint32))
    # every column line of both experts against the oracle
    log("column lines vs oracle")
    for e in range(w.num_experts):
        for c in range(w.k):
            _check_col_line(w, out, e, c)
    # sampled rows, including both ends of each expert
    rng = np.random.default_rng(61)
    r1 = int(w.splits[0])
    rows = [0, 1, r1 - 1, r1, w.sum_m - 1] + rng.integers(0, w.sum_m, 200).tolist()
    for r in rows:
        _check_row(w, out, r)
    # the graph-safe call on the same routing: byte-identical
    log("graph-safe at 2^24 rows")
    d_offs = torch.tensor(B.offsets_from_splits([int(v) for v in w.splits]), dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    gout = B.alloc_outputs(w.sum_m, w.k, w.num_experts, True, True, device="cuda:0")
    B.nvfp4_group_quantize_graphsafe(x, w.num_experts, d_offs, d_status, **gout)
    torch.cuda.synchronize()
    assert int(d_status.item()) == 0
    for key in dout:
        assert torch.equal(gout[key], dout[key]), key


def test_column_limit_k_2_to_22():
    log("generating 128 x 2^22")
    w = synth.max_k()
    log(f"quantize {w.name}")
    x, dout = _run(w)
    out = {key: t.cpu().numpy() for key, t in dout.items()}
    # every column amax: the max of |x| over the column (exact)
    want = _amax_from_bits(_abs_bits(w.x).max(axis=0))
    assert np.array_equal(out["col_amax"].view(np.uint32), want.view(np.uint32))
    # every row amax and sampled rows (4M elements each) against the oracle
    for r in range(w.sum_m):
        assert out["row_amax"][r] == O.row_amax(w.x, r), f"row_amax[{r}]"
    for r in (0, 1, 77, w.sum_m - 1):
        _check_row(w, out, r)
    # sampled column lines, including the last chunk
    rng = np.random.default_rng(71)
    cols = [0, 1, 255, 256, w.k - 256, w.k - 16, w.k - 1] + rng.integers(0, w.k, 200).tolist()
    for c in cols:
        _check_col_line(w, out, 0, c)
    # rowwise-only request (the fused pass does not cover this K: amax + cast)
    log("rowwise-only at K = 2^22")
    _, rout = _run(w, rowwise=True, columnwise=False)
    for key in ("row_amax", "row_data", "row_scale"):
        assert torch.equal(rout[key], dout[key]), key


@pytest.mark.parametrize("which", ["rows", "k"])
def test_mxfp4_at_the_limits(which):
    # 2^24 rows with K = 32 (MXFP4 blocks are 32 wide), or K = 2^22
    w = synth.max_rows(k=32) if which == "rows" else synth.max_k()
    log(f"mxfp4 cast {w.name}")
    dev = torch.device("cuda:0")
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    mx = B.alloc_mx_outputs(w.sum_m, w.k, device=dev)
    B.mxfp4_group_cast(x, [int(v) for v in w.splits], **mx)
    torch.cuda.synchronize()
    out = {key: t.cpu().numpy() for key, t in mx.items()}
    f32 = lambda bits: synth.bf16_bits_to_f32(np.ascontiguousarray(bits))
    rng = np.random.default_rng(81)
    for r in [0, w.sum_m - 1] + rng.integers(0, w.sum_m, 20).tolist():
        d, s = O.mx_encode_line(f32(w.x[r]))
        assert np.array_equal(out["row_data"][r], d) and np.array_equal(out["row_scale"][r], s), f"row {r}"
    offs = np.concatenate([[0], np.cumsum(w.splits)]).astype(np.int64)
    cols = list(range(w.k)) if w.k <= 32 else [0, 1, w.k - 1] + rng.integers(0, w.k, 50).tolist()
    for e in range(w.num_experts):
        r0, m = int(offs[e]), int(w.splits[e])
        for c in cols:
            d, s = O.mx_encode_line(f32(w.x[r0:r0 + m, c]))
            d0, s0 = w.k * r0 // 2 + c * (m // 2), w.k * r0 // 32 + c * (m // 32)
            assert np.array_equal(out["col_data"][d0:d0 + m // 2], d), f"col {e}, {c}"
            assert np.array_equal(out["col_scale"][s0:s0 + m // 32], s), f"col scale {e}, {c}"


@pytest.mark.parametrize("rows,k,splits", [(1 << 24, 16, [(1 << 24) - (1 << 17), 1 << 17]),
                                           (128, 1 << 22, [128])])
def test_dequant_at_the_limits(rows, k, splits):
    # seeded encoded inputs (every code byte, valid scale codes) sized at the limits
    n = rows * k
    log(f"dequant {rows} x {k}")
    data, scale = synth.random_encoded(91, n // 2)
    dev = torch.device("cuda:0")
    d_data, d_scale = torch.from_numpy(data).to(dev), torch.from_numpy(scale).to(dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    rng = np.random.default_rng(92)
    # rowwise: lines are rows of k elements
    ra = synth.random_amax(93, rows)
    B.nvfp4_group_dequant_rowwise(d_data.view(rows, k // 2), d_scale.view(rows, k // 16),
                                  torch.from_numpy(ra).to(dev), out.view(rows, k))
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(rows, k)
    for r in [0, rows - 1] + rng.integers(0, rows, 30).tolist():
        want = O.decode_line(data[r * k // 2:(r + 1) * k // 2], scale[r * k // 16:(r + 1) * k // 16], k, ra[r])
        assert np.array_equal(got[r].view(np.uint32), want.view(np.uint32)), f"row {r}"
    # columnwise: per expert k lines of M_e elements
    ca = synth.random_amax(94, len(splits) * k)
    B.nvfp4_group_dequant_columnwise(d_data, d_scale, torch.from_numpy(ca).to(dev), splits, k, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    offs = np.concatenate([[0], np.cumsum(splits)]).astype(np.int64)
    for e, m in enumerate(splits):
        r0 = int(offs[e])
        for c in [0, k - 1] + rng.integers(0, k, 10).tolist():
            base = k * r0 + c * m
            want = O.decode_line(data[base // 2:(base + m) // 2], scale[base // 16:(base + m) // 16], m,
                                 ca[e * k + c])
            assert np.array_equal(got[base:base + m].view(np.uint32), want.view(np.uint32)), f"col {e}, {c}"


def _values(data, scale, length):
    return O.block_values(data, scale, length)  # value(code) * value(S), exact in float64


def test_gemm_forward_at_k_2_to_22_exact():
    # sums of 2^22 products of 0, +-0.5, +-1: exact in fp32, so out == the
    # oracle's float64 product exactly
    k, n, rows = 1 << 22, 16, 128
    log("gemm forward k = 2^22")
    ad, as_, aa = synth.exact_nvfp4_lines(101, rows, k)
    bd, bs, ba = synth.exact_nvfp4_lines(102, n, k)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    out = torch.empty((rows, n), dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_gemm(dev(ad), dev(as_), dev(aa), dev(bd.reshape(1, n, -1)), dev(bs.reshape(1, n, -1)), dev(ba),
                       [rows], out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    vb = _values(bd, bs, k)
    for r in (0, 1, 64, rows - 1):
        want = _values(ad[r:r + 1], as_[r:r + 1], k) @ vb.T
        assert np.array_equal(got[r:r + 1], want), f"row {r}"


def test_gemm_forward_at_n_2_to_20_exact():
    k, n, rows = 128, 1 << 20, 128
    log("gemm forward n = 2^20")
    ad, as_, aa = synth.exact_nvfp4_lines(103, rows, k)
    bd, bs, ba = synth.exact_nvfp4_lines(104, n, k)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    out = torch.empty((rows, n), dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_gemm(dev(ad), dev(as_), dev(aa), dev(bd.reshape(1, n, -1)), dev(bs.reshape(1, n, -1)), dev(ba),
                       [rows], out)
    torch.cuda.synchronize()
    cols = np.array([0, 1, 255, 256, n - 256, n - 1] + np.random.default_rng(105).integers(0, n, 64).tolist())
    got = out[:, torch.from_numpy(cols).to("cuda:0")].cpu().numpy().astype(np.float64)
    want = _values(ad, as_, k) @ _values(bd[cols], bs[cols], k).T
    assert np.array_equal(got, want)


def test_gemm_wgrad_at_2_to_22_rows_exact():
    # one expert of 2^22 rows (the weight gradient's limit); every output
    m, n, k = 1 << 22, 16, 16
    log("gemm weight gradient, 2^22 rows")
    yd, ys, ya = synth.exact_nvfp4_lines(106, n, m)   # dY^T lines [n, m]
    xd, xs, xa = synth.exact_nvfp4_lines(107, k, m)   # X^T lines [k, m]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to("cuda:0")
    out = torch.empty((1, n, k), dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_gemm_wgrad(dev(yd), dev(ys), dev(ya), dev(xd), dev(xs), dev(xa), [m], n, k, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0].astype(np.float64)
    want = _values(yd, ys, m) @ _values(xd, xs, m).T
    assert np.array_equal(got, want)
