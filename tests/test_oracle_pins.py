"""Pins of the CPU oracle against what the format definitions and the
mathematics fix (no GPU).

What pins what:
  * E4M3FN conversion: format constants, every code round-trips, midpoints go
    to the even code, and a dense sweep of [0, 448] agrees with torch's own
    float32 -> float8_e4m3fn cast (a library routine that rounds to nearest
    even and agrees with saturation below 464).
  * E2M1 conversion: grid points, every midpoint (ties to even), neighbours of
    every midpoint, saturation and sign handling, and a dense sweep against
    the independent numpy brute force.
  * whole encode: closed-form round trips (inputs built as g * S * 2^j are
    reproduced bit for bit), hand-worked golden rows, the independent brute
    force on small tensors, and the half-gap error bound.
  * grouping: grouped call == per-expert loop, amax == numpy max, zero-row
    experts, empty input, argument rejection.
"""
import os

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------------- E4M3FN

def test_e4m3_format_constants(O):
    # OCP E4M3FN: bias 7, 3 mantissa bits, max finite 448 (0x7E), smallest
    # subnormal 2^-9, smallest normal 2^-6.
    assert O.e4m3_value(0x7E) == 448.0
    assert O.e4m3_value(0x01) == 2.0 ** -9
    assert O.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert O.e4m3_value(0x08) == 2.0 ** -6
    assert O.e4m3_value(0x38) == 1.0
    assert O.e4m3_value(0x30) == 0.5
    vals = [O.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_e4m3_codes_roundtrip_and_ties(O):
    vals = np.array([O.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
    assert (O.e4m3_encode(vals.astype(np.float32)) == np.arange(0x7F)).all()
    mids = 0.5 * (vals[:-1] + vals[1:])
    assert (mids.astype(np.float32).astype(np.float64) == mids).all()   # exact in fp32
    got = O.e4m3_encode(mids.astype(np.float32))
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert (got == want).all()
    up = np.nextafter(mids.astype(np.float32), np.float32(np.inf))
    dn = np.nextafter(mids.astype(np.float32), np.float32(0))
    assert (O.e4m3_encode(up) == lo + 1).all()
    assert (O.e4m3_encode(dn) == lo).all()


def test_e4m3_saturates(O):
    t = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, np.inf], dtype=np.float32)
    assert (O.e4m3_encode(t) == 0x7E).all()
    # just below 448: nearest is 448 above the 416/448 midpoint
    assert O.e4m3_encode(np.array([433.0], np.float32))[0] == 0x7E
    assert O.e4m3_encode(np.array([431.0], np.float32))[0] == 0x7D


def test_e4m3_sweep_matches_torch_cast(O):
    hi = int(f32_bits(448.0))
    bits = np.arange(0, hi + 1, 97, dtype=np.uint32)
    t = bits.view(np.float32)
    mine = O.e4m3_encode(t)
    ref = torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int32)
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, (t[bad[:5]], mine[bad[:5]], ref[bad[:5]])


def test_e4m3_matches_bruteforce(O, BF):
    rng = np.random.default_rng(11)
    t = np.concatenate([
        rng.uniform(0, 460, 20000), 2.0 ** rng.uniform(-14, 9, 20000),
    ]).astype(np.float32)
    assert (O.e4m3_encode(t) == BF.e4m3_encode(t)).all()


# ------------------------------------------------------------------- E2M1

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_grid_and_ties(O):
    for c, g in enumerate(GRID):
        assert O.e2m1_encode(np.array([g], np.float32))[0] == c
        assert O.e2m1_encode(np.array([-g], np.float32))[0] == c | 8
        assert O.e2m1_value(c) == g and O.e2m1_value(c | 8) == -g
    # midpoints and the even code each goes to
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for a, c in ties.items():
        v = np.array([a, -a], np.float32)
        assert O.e2m1_encode(v).tolist() == [c, c | 8]
        up = np.nextafter(np.float32(a), np.float32(np.inf))
        dn = np.nextafter(np.float32(a), np.float32(0))
        lo_code = [i for i, g in enumerate(GRID) if g < a][-1]
        assert O.e2m1_encode(np.array([up], np.float32))[0] == lo_code + 1
        assert O.e2m1_encode(np.array([dn], np.float32))[0] == lo_code


def test_e2m1_saturation_and_signs(O):
    v = np.array([6.0, 6.5, 7.0, 1e30, np.inf, -6.5, -np.inf, -0.0, -1e-40, 1e-40, -0.2],
                 dtype=np.float32)
    assert O.e2m1_encode(v).tolist() == [7, 7, 7, 7, 7, 15, 15, 8, 8, 0, 8]


def test_e2m1_sweep_matches_bruteforce(O, BF):
    bits = np.arange(0, int(f32_bits(7.0)), 1013, dtype=np.uint32)
    a = bits.view(np.float32)
    v = np.concatenate([a, -a])
    assert (O.e2m1_encode(v) == BF.e2m1_encode(v)).all()
    # monotone in the magnitude
    mag = O.e2m1_encode(a)
    assert (np.diff(mag) >= 0).all()


# ---------------------------------------------------------- block and line

def test_block_scale_zero_and_clamp(O):
    S, m = O.block_scale(np.array([0.0, 1.0], np.float32), np.array([0.0, 0.0], np.float32))
    assert S.tolist() == [0, 0] and m.tolist() == [0.0, 0.0]
    # tiny line scale: d = value(S) * s is so small that 1/d overflows and is clamped
    s = np.float32(2.0 ** -140)
    S, m = O.block_scale(np.array([6 * 448 * 2.0 ** -140], np.float32), np.array([s], np.float32))
    assert S[0] == 0x7E and m[0] == np.finfo(np.float32).max
    # a block whose scale underflows to E4M3 zero gets m = 0 (codes are signed zeros)
    S, m = O.block_scale(np.array([1e-3], np.float32), np.array([1.0], np.float32))
    assert S[0] == 0 and m[0] == 0.0


def _golden_row():
    xs, out = [], {}
    with open(os.path.join(GOLDEN, "worked_row_k64.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "x":
                xs += [int(v, 16) for v in vals]
            else:
                out[key] = [int(v, 16) for v in vals]
    x = np.array(xs, dtype=np.uint16)
    amax = np.array(out["amax"], dtype=np.uint32).view(np.float32)[0]
    return x, amax, np.array(out["data"], np.uint8), np.array(out["scale"], np.uint8)


def test_golden_worked_row(O, BF):
    x, amax, data, scale = _golden_row()
    assert x.size == 64
    xm = x.reshape(1, 64)
    assert O.row_amax(xm, 0) == amax
    d, s = O.cast_row(xm, 0, amax)
    assert d.tolist() == data.tolist()
    assert s.tolist() == scale.tolist()
    bd, bs = BF.encode_line(BF.bf16_to_f32(x), amax)
    assert bd.tolist() == data.tolist() and bs.tolist() == scale.tolist()


def test_golden_worked_column(O):
    # The same 64 values placed down column 0 of a one-expert 128 x 16 input:
    # the columnwise line of column 0 is the golden row followed by 64 zeros
    # (same line amax), every other column is all zero (amax 0 -> zero codes
    # and scales).  Rowwise, each row holds one value, so its line amax is
    # |x| and the value encodes to +-6 (code 7 | sign) with scale 448 (0x7E);
    # a row holding +-0 has amax 0, scale 0 and code sign<<3.
    x, amax, data, scale = _golden_row()
    X = np.zeros((128, 16), np.uint16)
    X[:64, 0] = x
    q = O.group_quantize(X, [128])
    assert q["col_amax"][0] == amax and (q["col_amax"][1:] == 0).all()
    cd = q["col_data"].reshape(16, 64)
    cs = q["col_scale"].reshape(16, 8)
    assert cd[0].tolist() == data.tolist() + [0] * 32
    assert cs[0].tolist() == scale.tolist() + [0] * 4
    assert (cd[1:] == 0).all() and (cs[1:] == 0).all()
    for r in range(128):
        v = int(X[r, 0])
        sign = 8 if v & 0x8000 else 0
        nonzero = (v & 0x7FFF) != 0
        want = (7 | sign) if nonzero else sign
        assert q["row_data"][r].tolist() == [want] + [0] * 7, r
        assert q["row_scale"][r].tolist() == [0x7E if nonzero else 0], r


def _closed_form_line(rng, n):
    """A line whose exact quantisation is known: s = 2^j, and each block holds
    g * S * 2^j with g on the E2M1 grid and one element at +-6 * S * 2^j, so
    t = S exactly; one block has S = 448, which makes A = 2688 * 2^j."""
    j = int(rng.integers(-20, 12))
    nb = n // 16
    codes = rng.integers(1, 0x7F, nb)       # every finite nonzero E4M3 code
    codes[rng.integers(0, nb)] = 0x7E
    grid = np.array(GRID, np.float64)
    out = np.empty(n, np.float64)
    for b in range(nb):
        e, f = codes[b] >> 3, codes[b] & 7
        S = f * 2.0 ** -9 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7)
        g = grid[rng.integers(0, 8, 16)] * rng.choice([-1.0, 1.0], 16)
        g[rng.integers(0, 16)] = 6.0 * rng.choice([-1.0, 1.0])
        out[16 * b:16 * (b + 1)] = g * S * 2.0 ** j
    return out.astype(np.float32), codes


def test_closed_form_roundtrip_rowwise(O):
    rng = np.random.default_rng(5)
    for _ in range(300):
        n = 16 * int(rng.integers(1, 12))
        L, codes = _closed_form_line(rng, n)
        # values are bf16-representable (<= 6 significant bits)
        assert (synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(L)) == L).all()
        A = np.float32(np.abs(L).max())
        d, s = O.encode_line(L, A)
        assert s.tolist() == codes.tolist()
        back = O.decode_line(d, s, n, A)
        assert (f32_bits(back) == f32_bits(L)).all()


def test_closed_form_roundtrip_both_directions(O):
    # every row block and every column block holds a +-6*448 element on the
    # r % 16 == c % 16 diagonal, so all line amaxes are 2688 (s = 1) and all
    # block scales are 448: both directions reproduce the input exactly.
    rng = np.random.default_rng(6)
    splits = [128, 256, 0, 128]
    M, K = 512, 96
    g = np.array(GRID)[rng.integers(0, 8, (M, K))] * rng.choice([-1.0, 1.0], (M, K))
    r, c = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    g[(r % 16) == (c % 16)] = 6.0 * rng.choice([-1.0, 1.0], int(((r % 16) == (c % 16)).sum()))
    Xf = (g * 448.0).astype(np.float32)
    X = synth.f32_to_bf16_bits(Xf)
    q = O.group_quantize(X, splits)
    assert (q["row_scale"] == 0x7E).all() and (q["col_scale"] == 0x7E).all()
    back_r = O.decode_rowwise(q["row_data"], q["row_scale"], q["row_amax"])
    back_c = O.decode_columnwise(q["col_data"], q["col_scale"], q["col_amax"], splits, K)
    assert (f32_bits(back_r) == f32_bits(Xf)).all()
    assert (f32_bits(back_c) == f32_bits(Xf)).all()


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("case", [
    ("tiny", None),
    ("rand", (7, [128, 0, 256], 48, "normal")),
    ("rand", (8, [256, 128], 80, "outliers")),
    ("rand", (9, [128, 128], 32, "sparse")),
    ("rand", (10, [0, 128, 0], 16, "student")),
    ("rand", (12, [128, 256], 64, "rowscale")),
])
def test_oracle_matches_bruteforce(O, BF, case):
    kind, args = case
    w = synth.tiny() if kind == "tiny" else synth.random_case(*args)
    q = O.group_quantize(w.x, w.splits)
    b = BF.group_quantize(w.x, w.splits)
    for key in ("row_amax", "col_amax"):
        assert (f32_bits(q[key]) == f32_bits(b[key])).all(), key
    for key in ("row_data", "row_scale", "col_data", "col_scale"):
        assert (q[key] == b[key]).all(), key


# ---------------------------------------------------------------- grouping

def test_amax_matches_numpy_and_invariants(O):
    w = synth.random_case(21, [128, 0, 384, 128], 112, "rowscale")
    ra, ca = O.group_amax(w.x, w.splits)
    xf = synth.bf16_bits_to_f32(w.x)
    assert (ra == np.abs(xf).max(axis=1)).all()
    r0 = 0
    for e, m in enumerate(w.splits):
        seg = ca[e * w.k:(e + 1) * w.k]
        if m == 0:
            assert (seg == 0).all()
        else:
            assert (seg == np.abs(xf[r0:r0 + m]).max(axis=0)).all()
            assert seg.max() == ra[r0:r0 + m].max()
        r0 += m


def test_grouped_equals_per_expert_loop(O):
    w = synth.random_case(22, [256, 0, 128, 384, 0], 48, "outliers")
    q = O.group_quantize(w.x, w.splits)
    r0 = 0
    k = w.k
    for e, m in enumerate(w.splits):
        m = int(m)
        if m == 0:
            continue
        one = O.group_quantize(w.x[r0:r0 + m], [m])
        assert (one["row_data"] == q["row_data"][r0:r0 + m]).all()
        assert (one["row_scale"] == q["row_scale"][r0:r0 + m]).all()
        assert (one["col_amax"] == q["col_amax"][e * k:(e + 1) * k]).all()
        assert (one["col_data"] == q["col_data"][k * r0 // 2:k * (r0 + m) // 2]).all()
        assert (one["col_scale"] == q["col_scale"][k * r0 // 16:k * (r0 + m) // 16]).all()
        r0 += m


def test_columnwise_is_rowwise_of_transpose(O):
    # By definition the columnwise output of expert e is the rowwise output of
    # X_e transposed, with the per-column amax as the line amax.
    w = synth.random_case(23, [256], 32, "normal")
    q = O.group_quantize(w.x, w.splits)
    xt = np.ascontiguousarray(w.x.T)            # (32, 256)
    for c in range(w.k):
        d, s = O.cast_row(xt, c, q["col_amax"][c])
        assert (d == q["col_data"].reshape(w.k, -1)[c]).all()
        assert (s == q["col_scale"].reshape(w.k, -1)[c]).all()


def test_half_gap_error_bound(O):
    # |x^ - x| <= gap/2 * d (gap: 0.5 below 2, 1 below 4, else 2) for blocks
    # with a normal E4M3 scale; for subnormal scales saturation may add up to
    # b - 6d.  Relative slack 2^-16 covers the fp32 roundings of m, x*m, x^.
    w = synth.random_case(24, [128, 256], 64, "rowscale")
    q = O.group_quantize(w.x, w.splits)
    xf = synth.bf16_bits_to_f32(w.x).astype(np.float64)
    back = O.decode_rowwise(q["row_data"], q["row_scale"], q["row_amax"]).astype(np.float64)
    s = (q["row_amax"] / np.float32(2688.0)).astype(np.float64)
    Sval = np.array([O.e4m3_value(c) for c in range(0x7F)])[q["row_scale"]]     # (M, K/16)
    d = np.repeat(Sval, 16, axis=1) * s[:, None]
    y = np.abs(xf) / np.where(d > 0, d, 1)
    gap = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    b = np.repeat(np.abs(xf).reshape(xf.shape[0], -1, 16).max(axis=2), 16, axis=1)
    normal = np.repeat(q["row_scale"] >= 8, 16, axis=1)
    bound = np.where(normal, 0.5 * gap * d, np.maximum(0.5 * gap * d, b - 6 * d))
    err = np.abs(back - xf)
    assert (err <= bound * (1 + 2.0 ** -16) + 1e-45).all()
    assert normal.mean() > 0.99


def test_edge_cases(O):
    # empty input
    x = np.zeros((0, 32), np.uint16)
    q = O.group_quantize(x, [0, 0])
    assert q["row_amax"].size == 0 and (q["col_amax"] == 0).all() and q["col_data"].size == 0
    # all zero, with negative zeros: codes keep the sign, scales 0
    x = np.zeros((128, 16), np.uint16)
    x[::2, 3] = 0x8000
    q = O.group_quantize(x, [128])
    assert (q["row_scale"] == 0).all() and (q["col_scale"] == 0).all()
    assert (q["row_data"][::2, 1] == 0x80).all() and (q["row_data"][1::2] == 0).all()
    # single nonzero element per block: encodes as +-6 at scale 448
    x = np.zeros((128, 32), np.uint16)
    x[:, 5] = 0xC0A0   # -5.0
    q = O.group_quantize(x, [128])
    assert (q["row_data"][:, 2] == 0xF0).all() and (q["row_scale"][:, 0] == 0x7E).all()
    assert (q["row_scale"][:, 1] == 0).all()


def test_rejects_bad_arguments(O):
    x = np.zeros((256, 32), np.uint16)
    for splits in ([100, 156], [128, 0], [-128, 384], [128, 256]):
        with pytest.raises(ValueError):
            O.group_amax(x, splits)
    with pytest.raises(ValueError):
        O.group_amax(np.zeros((128, 24), np.uint16), [128])
