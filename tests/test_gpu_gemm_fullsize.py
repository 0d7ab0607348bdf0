"""The row-scaled grouped GEMM at the benchmark's shapes and launch
configuration: the expert-share rows (32 experts, Zipf routing, sum_M=65536,
K=7168) times per-expert weights of 2048 output features, forward and weight
gradient.  Operands are seeded random NVFP4 bytes (every code byte, finite
E4M3 scales, positive amax) drawn on the host; sampled outputs are compared
with the oracle's float64 dot product of the decoded lines, within the
rounding bound derived in test_gpu_gemm.py.  A hipGraph capture of the
graph-safe forward call is replayed under new routing and compared with the
host-split call each time.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import log

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
E, K, M, N = 32, 7168, 65536, 2048


def _operand(rng, lines, length):
    data = rng.integers(0, 256, (lines, length // 2), dtype=np.uint8)
    scale = rng.integers(0x20, 0x50, (lines, length // 16), dtype=np.uint8)
    return data, scale


def _dot(da, sa, aa, db, sb, ab, length):
    va = O.block_values(da[None], sa[None], length)[0]
    vb = O.block_values(db[None], sb[None], length)[0]
    p = va * vb
    s = float(aa) / 2688.0 * float(ab) / 2688.0
    return float(p.sum()) * s, float(np.abs(p).sum()) * abs(s)


def _check(got, want, bound, L, what):
    lim = (2 * L + 8) * U * bound + 1e-30
    assert abs(got - want) <= lim, f"{what}: gpu {got} oracle {want} (bound {lim})"


def test_forward_expert_share_sampled():
    rng = np.random.default_rng(101)
    splits = [int(v) for v in synth.zipf_splits(np.random.default_rng(3), E, M)]
    ad, as_ = _operand(rng, M, K)
    aa = rng.uniform(0.25, 4.0, M).astype(np.float32)
    bd, bs = _operand(rng, E * N, K)
    ba = rng.uniform(0.25, 4.0, E * N).astype(np.float32)
    log(f"gemm fwd full size sum_m={M} n={N} k={K}")
    dev = lambda a: torch.from_numpy(a).to("cuda:0")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_gemm(dev(ad), dev(as_), dev(aa), dev(bd.reshape(E, N, -1)), dev(bs.reshape(E, N, -1)), dev(ba),
                       splits, out)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(splits)])
    rows = rng.integers(0, M, 48).tolist() + [int(o) for o in offs[1:] - 1 if o > 0]
    cols = rng.integers(0, N, len(rows)).tolist()
    got = out.cpu().numpy()
    for r, j in zip(rows, cols):
        e = int(np.searchsorted(offs, r, side="right") - 1)
        while splits[e] == 0:
            e += 1
        want, bound = _dot(ad[r], as_[r], aa[r], bd[e * N + j], bs[e * N + j], ba[e * N + j], K)
        _check(float(got[r, j]), want, bound, K, f"out[{r}, {j}] (expert {e})")
    assert np.isfinite(got).all()


def test_wgrad_expert_share_sampled():
    rng = np.random.default_rng(102)
    splits = [int(v) for v in synth.zipf_splits(np.random.default_rng(3), E, M)]
    yd, ys = _operand(rng, 1, M * N)
    ya = rng.uniform(0.25, 4.0, E * N).astype(np.float32)
    xd, xs = _operand(rng, 1, M * K)
    xa = rng.uniform(0.25, 4.0, E * K).astype(np.float32)
    yd, ys, xd, xs = yd[0], ys[0], xd[0], xs[0]
    log(f"gemm wgrad full size sum_m={M} n={N} k={K}")
    dev = lambda a: torch.from_numpy(a).to("cuda:0")
    out = torch.empty((E, N, K), dtype=torch.float32, device="cuda:0")
    B.nvfp4_group_gemm_wgrad(dev(yd), dev(ys), dev(ya), dev(xd), dev(xs), dev(xa), splits, N, K, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    offs = np.concatenate([[0], np.cumsum(splits)])
    for e, m in enumerate(splits):
        if m == 0:
            assert (got[e] == 0).all()
            continue
        r0 = int(offs[e])
        for i, j in zip(rng.integers(0, N, 2).tolist(), rng.integers(0, K, 2).tolist()):
            la = slice((N * r0 + i * m) // 2, (N * r0 + (i + 1) * m) // 2)
            sa = slice((N * r0 + i * m) // 16, (N * r0 + (i + 1) * m) // 16)
            lb = slice((K * r0 + j * m) // 2, (K * r0 + (j + 1) * m) // 2)
            sb = slice((K * r0 + j * m) // 16, (K * r0 + (j + 1) * m) // 16)
            want, bound = _dot(yd[la], ys[sa], ya[e * N + i], xd[lb], xs[sb], xa[e * K + j], m)
            _check(float(got[e, i, j]), want, bound, m, f"dW[{e}, {i}, {j}] (M_e={m})")


def test_forward_graph_replays_under_new_routing():
    # one capture of the graph-safe call, replayed with new routing written to
    # the device offsets; every replay equals the host-split call bit for bit
    rng = np.random.default_rng(103)
    m_cap, n, k, e_n = 8192, 512, 1024, 8
    ad, as_ = _operand(rng, m_cap, k)
    aa = rng.uniform(0.25, 4.0, m_cap).astype(np.float32)
    bd, bs = _operand(rng, e_n * n, k)
    ba = rng.uniform(0.25, 4.0, e_n * n).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    ta = (dev(ad), dev(as_), dev(aa))
    tb = (dev(bd.reshape(e_n, n, -1)), dev(bs.reshape(e_n, n, -1)), dev(ba))
    d_offs = torch.zeros(e_n, dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    out = torch.zeros((m_cap, n), dtype=torch.float32, device="cuda:0")
    def route(units):
        w = rng.uniform(0.1, 1.0, e_n) * (rng.uniform(0, 1, e_n) > 0.25)
        w[rng.integers(0, e_n)] = 1.0
        return synth.largest_remainder(w, units) * 128
    routes = [route(m_cap // 128 - 3 * i) for i in range(4)]
    d_offs.copy_(torch.tensor(B.offsets_from_splits(routes[0]), dtype=torch.int32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.nvfp4_group_gemm_graphsafe(*ta, *tb, d_offs, out, d_status)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.nvfp4_group_gemm_graphsafe(*ta, *tb, d_offs, out, d_status)
    torch.cuda.synchronize()
    for i, sp in enumerate(routes):
        sp = [int(v) for v in sp]
        total = sum(sp)
        d_offs.copy_(torch.tensor(B.offsets_from_splits(sp), dtype=torch.int32))
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        ref = torch.empty((total, n), dtype=torch.float32, device="cuda:0")
        B.nvfp4_group_gemm(ta[0][:total], ta[1][:total], ta[2][:total], *tb, sp, ref)
        torch.cuda.synchronize()
        assert int(d_status.item()) == 0
        assert torch.equal(out[:total].view(torch.int32), ref.view(torch.int32)), f"replay {i}"
        assert (out[total:] == 0).all(), f"replay {i} wrote rows beyond the routed total"
        log(f"replay {i}: routed {total} of {m_cap} rows, byte-identical")
