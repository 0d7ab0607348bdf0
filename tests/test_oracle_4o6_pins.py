"""Pins of the oracle's four-over-six block scaling (the recipe named on the
torchtitan converter page, "[NVFP4 4over6] Add the grouped-experts
four-over-six converter", Summary and Review pass; the selection rule is the
reading stated in the oracle: each block encoded with its amax mapped to 6
and to 4, the smaller error kept).

What pins it, other than its own formula:
- a hand-worked golden row (tests/golden/worked_4o6_k48.txt, derivation in
  the file);
- closed forms: blocks whose values lie on the 4-scaled grid are reproduced
  exactly and choose 4, blocks on the 6-scaled grid are reproduced exactly
  and choose 6;
- with bound 448 the k = 6 candidate is the plain recipe's block step, so
  every block choosing 6 has the plain recipe's bytes and every block's
  squared error is at most the plain recipe's;
- an independent numpy brute force (nearest-value search) gives the same
  bytes and choices on random lines for both error modes and three bounds;
- the chosen candidate's error stays within half an E2M1 gap per element;
- grouped equals the per-expert loop, and columnwise equals rowwise of the
  transpose.
Matching the bytes of the published method's own implementation is not
pinned: no such output is available here.
"""
import os

import numpy as np
import pytest

from nvfp4_block_scaled_group_amd import synth
from oracle import bruteforce as BF
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def _golden():
    xs, out = [], {}
    with open(os.path.join(GOLDEN, "worked_4o6_k48.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "x":
                xs += [int(v, 16) for v in vals]
            elif key == "pick":
                out[key] = [int(v) for v in vals]
            else:
                out[key] = [int(v, 16) for v in vals]
    x = np.array(xs, dtype=np.uint16)
    amax = np.array(out["amax"], dtype=np.uint32).view(np.float32)[0]
    return x, amax, out


def test_golden_worked_row():
    x, amax, g = _golden()
    L = BF.bf16_to_f32(x)
    assert O.row_amax(x.reshape(1, -1), 0) == amax
    d, s, p = O.encode_line_4o6(L, amax, 256, O.ERR_MSE)
    assert d.tolist() == g["data"] and s.tolist() == g["scale"] and p.tolist() == g["pick"]
    bd, bs, bp = BF.encode_line_4o6(L, amax, 256, 0)
    assert bd.tolist() == g["data"] and bs.tolist() == g["scale"] and bp.tolist() == g["pick"]
    # the kept encodings of blocks 0 and 1 are exact: dequantised == input
    dq = O.decode_line_b(d, s, L.size, amax, 256)
    assert np.array_equal(dq[:32], L[:32])


GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.mark.parametrize("seed", range(8))
def test_closed_form_blocks_on_each_grid(seed):
    # line scale s = 2^j with A = 6*bound*2^j; blocks g*S*s with the largest g
    # = 4 (choose 4, exact) or = 6 (choose 6, exact), S a power of two so
    # that m = 1/d is exact
    rng = np.random.default_rng(seed)
    bound = 256
    j = int(rng.integers(-20, 20))
    s = 2.0 ** j
    A = 6 * bound * s
    blocks, want = [], []
    # block 0 carries the line amax: g_max = 6 with S = bound (b = 6*bound*s = A)
    for top, S in [(6, bound)] + [(int(rng.choice([4, 6])), 2.0 ** int(rng.integers(-6, 8))) for _ in range(5)]:
        g = rng.choice(GRID[GRID <= top], 16) * rng.choice([-1, 1], 16)
        g[int(rng.integers(0, 16))] = top
        blocks.append(g * S * s)
        want.append(top)
    L = np.concatenate(blocks).astype(np.float32)
    assert np.abs(L).max() == A
    for mode in (O.ERR_MSE, O.ERR_MAE):
        d, sc, p = O.encode_line_4o6(L, A, bound, mode)
        assert p.tolist() == [4 if t == 4 else 6 for t in want]
        assert np.array_equal(O.decode_line_b(d, sc, L.size, A, bound), L)


def _lines(seed, n_lines=60, k=64):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_lines):
        kind = i % 4
        v = rng.standard_normal(k).astype(np.float32)
        if kind == 1:
            v *= np.float32(np.exp(rng.standard_normal() * 4))
        elif kind == 2:
            v[rng.random(k) < 0.05] *= 100
        elif kind == 3:
            v = (rng.standard_t(3, k) * 1e-3).astype(np.float32)
        v = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v))
        out.append(v)
    return out


@pytest.mark.parametrize("bound", [448, 256, 100])
@pytest.mark.parametrize("mode", [0, 1])
def test_bruteforce_agrees(bound, mode):
    for L in _lines(bound * 10 + mode):
        A = float(np.abs(L).max())
        d, s, p = O.encode_line_4o6(L, A, bound, mode)
        bd, bs, bp = BF.encode_line_4o6(L, A, bound, mode)
        assert np.array_equal(d, bd) and np.array_equal(s, bs) and np.array_equal(p, bp)


def _sq_err(L, dq):
    return (np.asarray(L, np.float64) - np.asarray(dq, np.float64)) ** 2


def test_bound_448_candidate_six_is_the_plain_recipe():
    picks4 = 0
    for L in _lines(7, n_lines=80):
        A = float(np.abs(L).max())
        d, s, p = O.encode_line_4o6(L, A, 448, O.ERR_MSE)
        pd, ps = O.encode_line(L, A)
        dq = O.decode_line_b(d, s, L.size, A, 448)
        pq = O.decode_line(pd, ps, L.size, A)
        for j in range(L.size // 16):
            if p[j] == 6:
                assert s[j] == ps[j] and np.array_equal(d[8 * j:8 * j + 8], pd[8 * j:8 * j + 8])
            else:
                picks4 += 1
            # four-over-six never does worse than the plain recipe on a block
            assert _sq_err(L[16 * j:16 * j + 16], dq[16 * j:16 * j + 16]).sum() <= \
                _sq_err(L[16 * j:16 * j + 16], pq[16 * j:16 * j + 16]).sum() * (1 + 1e-6) + 1e-30
    assert picks4 > 0  # the k = 4 candidate does win on some blocks


def test_error_modes_both_decide():
    # the two error measures disagree on some blocks, and each mode's choice
    # matches the brute force there
    differ = 0
    for L in _lines(11, n_lines=200, k=16):
        A = float(np.abs(L).max())
        p0 = O.encode_line_4o6(L, A, 256, 0)[2][0]
        p1 = O.encode_line_4o6(L, A, 256, 1)[2][0]
        differ += int(p0 != p1)
        assert p0 == BF.encode_line_4o6(L, A, 256, 0)[2][0]
        assert p1 == BF.encode_line_4o6(L, A, 256, 1)[2][0]
    assert differ > 0


def test_half_gap_error_bound_of_the_kept_candidate():
    gap = lambda q: np.where(np.abs(q) < 2, 0.5, np.where(np.abs(q) < 4, 1.0, 2.0))
    for L in _lines(13, n_lines=80):
        A = float(np.abs(L).max())
        d, sc, p = O.encode_line_4o6(L, A, 256, O.ERR_MSE)
        s = float(O.line_scale_b(A, 256))
        dq = O.decode_line_b(d, sc, L.size, A, 256).astype(np.float64)
        codes = np.empty(L.size, np.int64)
        codes[0::2], codes[1::2] = d & 15, d >> 4
        q = np.array([O.e2m1_value(c) for c in codes])
        for j in range(L.size // 16):
            Sv = O.e4m3_value(int(sc[j]))
            if Sv < 2.0 ** -6 or Sv == 0:
                continue  # subnormal scale: the plain bound does not apply
            dd = Sv * s
            err = np.abs(L[16 * j:16 * j + 16] - dq[16 * j:16 * j + 16])
            assert (err <= 0.5 * gap(q[16 * j:16 * j + 16]) * dd * (1 + 2.0 ** -20) + 0.4 * dd * (
                np.abs(q[16 * j:16 * j + 16]) == 6)).all()


def test_zero_block_and_zero_line():
    L = np.zeros(32, np.float32)
    d, s, p = O.encode_line_4o6(L, 0.0, 256, O.ERR_MSE)
    assert (d == 0).all() and (s == 0).all() and (p == 6).all()


def test_grouped_equals_per_expert_loop_and_transpose():
    w = synth.random_case(91, [256, 0, 128, 384], 80, "rowscale")
    full = O.group_quantize_4o6(w.x, w.splits, 256, O.ERR_MSE)
    offs = np.concatenate([[0], np.cumsum(w.splits)]).astype(int)
    k = w.k
    for e, m in enumerate(w.splits):
        lo, hi = offs[e], offs[e + 1]
        part = O.group_quantize_4o6(np.ascontiguousarray(w.x[lo:hi]), [m], 256, O.ERR_MSE)
        assert np.array_equal(part["row_data"], full["row_data"][lo:hi])
        assert np.array_equal(part["row_scale"], full["row_scale"][lo:hi])
        assert np.array_equal(part["col_data"], full["col_data"][k * lo // 2:k * hi // 2])
        assert np.array_equal(part["col_scale"], full["col_scale"][k * lo // 16:k * hi // 16])
        if m:
            # columnwise == rowwise cast of the transposed expert with the column amax as line amax
            xt = BF.bf16_to_f32(w.x[lo:hi]).T
            for c in range(0, k, 7):
                d, s, _ = O.encode_line_4o6(xt[c], full["col_amax"][e * k + c], 256, O.ERR_MSE)
                assert np.array_equal(d, full["col_data"][k * lo // 2 + c * (m // 2): k * lo // 2 + (c + 1) * (m // 2)])
                assert np.array_equal(s, full["col_scale"][k * lo // 16 + c * (m // 16): k * lo // 16 + (c + 1) * (m // 16)])


def test_rejects_bad_knobs():
    L = np.ones(16, np.float32)
    with pytest.raises(ValueError):
        O.encode_line_4o6(L, 1.0, 0, 0)
    with pytest.raises(ValueError):
        O.encode_line_4o6(L, 1.0, 449, 0)
    with pytest.raises(ValueError):
        O.encode_line_4o6(L, 1.0, 256, 2)
