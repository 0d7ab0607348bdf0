"""Pins of the oracle's row-scaled grouped GEMM (no GPU).

The GEMM consumes the cast's outputs (TransformerEngine PR 2931 page: the
GEMM runs on the block-scaled FP4 operands and its fp32 rows are then scaled
by the row amax; PR 3324 page: the weight gradient is an NT GEMM per expert
on the columnwise operands).  Its oracle is the plain product of the
dequantised operands.  What pins it:
  * closed form: operands built so that the cast reproduces them exactly
    (every block holds a +-6 element, so each block scale is exact), whose
    GEMM is then X @ W_e^T (forward) or dY_e^T @ X_e (weight gradient) of the
    original matrices, computed here in float64 without any rounding;
  * an independent brute force on tiny operands: a pure-Python triple loop
    with its own E2M1 table and E4M3 formula, taken from the format
    definitions;
  * grouped == per-expert loop; the weight-gradient form with its operands
    swapped gives the transpose; experts without rows give zeros.
"""
import numpy as np
import pytest

from nvfp4_block_scaled_group_amd import synth

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3(code):
    e, f = code >> 3, code & 7
    return f * 2.0 ** -9 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7)


def _exact_line(rng, n, scale_codes):
    """A line of n values g * S_b * 2^j (g on the E2M1 grid, one +-6 per
    block, one block with S = 448) that the cast reproduces exactly."""
    j = int(rng.integers(-3, 4))
    nb = n // 16
    codes = rng.choice(scale_codes, nb)
    codes[rng.integers(0, nb)] = 0x7E
    out = np.empty(n)
    for b in range(nb):
        g = np.array(GRID)[rng.integers(0, 8, 16)] * rng.choice([-1.0, 1.0], 16)
        g[rng.integers(0, 16)] = 6.0 * rng.choice([-1.0, 1.0])
        out[16 * b:16 * (b + 1)] = g * _e4m3(int(codes[b])) * 2.0 ** j
    return out


def _quantize_rows(O, M):
    """Row-scaled NVFP4 of each row of M (float64 values that are exact in
    fp32): (data, scale, amax)."""
    rows, n = M.shape
    data = np.empty((rows, n // 2), np.uint8)
    scale = np.empty((rows, n // 16), np.uint8)
    amax = np.empty(rows, np.float32)
    for r in range(rows):
        L = M[r].astype(np.float32)
        amax[r] = np.abs(L).max()
        data[r], scale[r] = O.encode_line(L, amax[r])
    return data, scale, amax


# narrow scale exponents keep every dot product below exactly representable
# in float64 (at most ~50 significant bits)
SCALE_CODES = np.arange(0x28, 0x50)


def test_forward_closed_form(O):
    rng = np.random.default_rng(31)
    splits, n, k = [128, 0, 256, 128], 48, 96
    E, sum_m = len(splits), sum(splits)
    X = np.stack([_exact_line(rng, k, SCALE_CODES) for _ in range(sum_m)])
    W = np.stack([_exact_line(rng, k, SCALE_CODES) for _ in range(E * n)])
    xa = _quantize_rows(O, X)
    wb = _quantize_rows(O, W)
    # the cast reproduces the operands exactly
    assert (O.block_values(xa[0], xa[1], k) * (xa[2].astype(np.float64) / 2688.0)[:, None] == X).all()
    out, bound = O.group_gemm(*xa, wb[0].reshape(E, n, k // 2), wb[1].reshape(E, n, k // 16), wb[2],
                              splits, n, k)
    r0 = 0
    for e, m in enumerate(splits):
        want = X[r0:r0 + m] @ W[e * n:(e + 1) * n].T
        assert (out[r0:r0 + m] == want).all(), e
        assert (bound[r0:r0 + m] == np.abs(X[r0:r0 + m]) @ np.abs(W[e * n:(e + 1) * n]).T).all()
        r0 += m


def _bruteforce_forward(a_data, a_scale, a_amax, b_data, b_scale, b_amax, splits, n, k):
    def val(data, scale, r, t):
        byte = int(data[r][t // 2])
        code = byte & 15 if t % 2 == 0 else byte >> 4
        mag = GRID[code & 7] * _e4m3(int(scale[r][t // 16]))
        return -mag if code & 8 else mag
    out = [[0.0] * n for _ in range(sum(splits))]
    r0 = 0
    for e, m in enumerate(splits):
        for r in range(r0, r0 + m):
            for j in range(n):
                bj = e * n + j
                acc = 0.0
                for t in range(k):
                    acc += val(a_data, a_scale, r, t) * val(b_data, b_scale, bj, t)
                out[r][j] = acc * (float(a_amax[r]) / 2688.0) * (float(b_amax[bj]) / 2688.0)
        r0 += m
    return np.array(out)


def test_forward_matches_bruteforce(O):
    rng = np.random.default_rng(32)
    splits, n, k = [2, 0, 3], 5, 32     # the oracle does not need 128-row groups
    E, sum_m = len(splits), sum(splits)
    a_data = rng.integers(0, 256, (sum_m, k // 2), dtype=np.uint8)
    a_scale = rng.integers(0, 0x7F, (sum_m, k // 16), dtype=np.uint8)
    a_amax = rng.uniform(0.01, 100, sum_m).astype(np.float32)
    b_data = rng.integers(0, 256, (E * n, k // 2), dtype=np.uint8)
    b_scale = rng.integers(0, 0x7F, (E * n, k // 16), dtype=np.uint8)
    b_amax = rng.uniform(0.01, 100, E * n).astype(np.float32)
    out, _ = O.group_gemm(a_data, a_scale, a_amax, b_data.reshape(E, n, -1), b_scale.reshape(E, n, -1), b_amax,
                          splits, n, k)
    want = _bruteforce_forward(a_data, a_scale, a_amax, b_data, b_scale, b_amax, splits, n, k)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-300)


def test_forward_grouped_equals_per_expert(O):
    rng = np.random.default_rng(33)
    splits, n, k = [128, 256, 0, 128], 32, 64
    E, sum_m = len(splits), sum(splits)
    a = (rng.integers(0, 256, (sum_m, k // 2), dtype=np.uint8), rng.integers(0, 0x7F, (sum_m, k // 16), dtype=np.uint8),
         rng.uniform(0.1, 10, sum_m).astype(np.float32))
    b = (rng.integers(0, 256, (E, n, k // 2), dtype=np.uint8), rng.integers(0, 0x7F, (E, n, k // 16), dtype=np.uint8),
         rng.uniform(0.1, 10, E * n).astype(np.float32))
    out, _ = O.group_gemm(*a, *b, splits, n, k)
    r0 = 0
    for e, m in enumerate(splits):
        if m:
            one, _ = O.group_gemm(a[0][r0:r0 + m], a[1][r0:r0 + m], a[2][r0:r0 + m], b[0][e:e + 1], b[1][e:e + 1],
                                  b[2][e * n:(e + 1) * n], [m], n, k)
            assert (one == out[r0:r0 + m]).all(), e
        r0 += m


def _exact_both_directions(rng, M, C):
    """(M, C) values whose rowwise and columnwise casts are both exact: a
    +-6*448 element on the r % 16 == c % 16 diagonal of every block."""
    g = np.array(GRID)[rng.integers(0, 8, (M, C))] * rng.choice([-1.0, 1.0], (M, C))
    r, c = np.meshgrid(np.arange(M), np.arange(C), indexing="ij")
    diag = (r % 16) == (c % 16)
    g[diag] = 6.0 * rng.choice([-1.0, 1.0], int(diag.sum()))
    return g * 448.0


def test_wgrad_closed_form_and_swap(O):
    rng = np.random.default_rng(34)
    splits, n, k = [128, 0, 256], 32, 48
    E = len(splits)
    dY = _exact_both_directions(rng, sum(splits), n)
    X = _exact_both_directions(rng, sum(splits), k)
    qy = O.group_quantize(synth.f32_to_bf16_bits(dY.astype(np.float32)), splits)
    qx = O.group_quantize(synth.f32_to_bf16_bits(X.astype(np.float32)), splits)
    out, bound = O.group_gemm_wgrad(qy["col_data"], qy["col_scale"], qy["col_amax"],
                                    qx["col_data"], qx["col_scale"], qx["col_amax"], splits, n, k)
    assert out.shape == (E, n, k)
    r0 = 0
    for e, m in enumerate(splits):
        want = dY[r0:r0 + m].T @ X[r0:r0 + m]
        assert (out[e] == want).all(), e
        assert (bound[e] == np.abs(dY[r0:r0 + m]).T @ np.abs(X[r0:r0 + m])).all()
        if m == 0:
            assert (out[e] == 0).all()
        r0 += m
    swapped, _ = O.group_gemm_wgrad(qx["col_data"], qx["col_scale"], qx["col_amax"],
                                    qy["col_data"], qy["col_scale"], qy["col_amax"], splits, k, n)
    assert (swapped == out.transpose(0, 2, 1)).all()


@pytest.mark.parametrize("seed", [35, 36])
def test_gemm_of_cast_close_to_gemm_of_input(O, seed):
    # the GEMM of the quantised operands differs from the GEMM of the inputs
    # by at most the sum of the per-element quantisation errors, each within
    # its block's half-gap bound (|x^ - x| <= 0.5 * d * 2 for |x| <= 6d)
    rng = np.random.default_rng(seed)
    splits, n, k = [128, 128], 16, 64
    X = rng.standard_normal((sum(splits), k)).astype(np.float32)
    X = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(X))
    W = rng.standard_normal((2 * n, k)).astype(np.float32)
    W = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(W))
    xa = _quantize_rows(O, X.astype(np.float64))
    wb = _quantize_rows(O, W.astype(np.float64))
    out, _ = O.group_gemm(*xa, wb[0].reshape(2, n, -1), wb[1].reshape(2, n, -1), wb[2], splits, n, k)
    Xh = O.block_values(xa[0], xa[1], k) * (xa[2].astype(np.float64) / 2688)[:, None]
    Wh = O.block_values(wb[0], wb[1], k) * (wb[2].astype(np.float64) / 2688)[:, None]
    ex, ew = np.abs(Xh - X), np.abs(Wh - W)
    r0 = 0
    for e, m in enumerate(splits):
        Xe, We = X[r0:r0 + m].astype(np.float64), W[e * n:(e + 1) * n].astype(np.float64)
        err = np.abs(out[r0:r0 + m] - Xe @ We.T)
        lim = ex[r0:r0 + m] @ np.abs(We).T + np.abs(Xe) @ ew[e * n:(e + 1) * n].T + ex[r0:r0 + m] @ ew[e * n:(e + 1) * n].T
        assert (err <= lim * (1 + 1e-9)).all()
        r0 += m
