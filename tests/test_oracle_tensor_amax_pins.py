"""Pins of the oracle's per-tensor amax (row scaling off: every line of an
expert takes the expert's max |x|; the reading of the row_scaled knob on the
torchtitan converter page, "[NVFP4 4over6] Add the grouped-experts
four-over-six converter", Summary and Review pass, and of the per-tensor
amax the per-token page, "Implement per-token NVFP4 fprop recipe",
Description, says the per-row one replaces).

Pinned to: numpy's max over each expert's slice (an independent
computation), the maxima of the per-row and per-column amax, empty and
all-zero experts, and closed forms: with every line of an expert on one
scale, inputs g * value(S) * s on the grids are reproduced exactly by the
plain and the four-over-six casts."""
import numpy as np
import pytest

from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _case(seed, splits, k, dist="rowscale"):
    return synth.random_case(seed, splits, k, dist)


@pytest.mark.parametrize("seed,splits,k", [(1, [128, 0, 256], 48), (2, [384, 128, 128], 272), (3, [0, 0, 128], 16)])
def test_equals_numpy_max_per_expert(seed, splits, k):
    w = _case(seed, splits, k)
    ra, ca = O.group_amax_tensor(w.x, splits)
    xf = np.abs(synth.bf16_bits_to_f32(w.x))
    offs = np.concatenate([[0], np.cumsum(splits)]).astype(int)
    for e, m in enumerate(splits):
        want = np.float32(xf[offs[e]:offs[e + 1]].max()) if m else np.float32(0.0)
        assert (ca[e * k:(e + 1) * k] == want).all()
        assert (ra[offs[e]:offs[e + 1]] == want).all()


def test_is_the_max_of_the_line_amax():
    splits, k = [256, 128, 0, 384], 80
    w = _case(4, splits, k, "outliers")
    ra, ca = O.group_amax(w.x, splits)
    ta, tc = O.group_amax_tensor(w.x, splits)
    offs = np.concatenate([[0], np.cumsum(splits)]).astype(int)
    for e, m in enumerate(splits):
        if m == 0:
            assert (tc[e * k:(e + 1) * k] == 0).all()
            continue
        assert (ta[offs[e]:offs[e + 1]] == ra[offs[e]:offs[e + 1]].max()).all()
        assert (tc[e * k:(e + 1) * k] == ca[e * k:(e + 1) * k].max()).all()


def test_directions_and_zero_expert():
    splits, k = [128, 128], 32
    x = np.zeros((256, k), dtype=np.uint16)
    x[200, 5] = synth.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]
    ra, ca = O.group_amax_tensor(x, splits)
    assert (ra[:128] == 0).all() and (ra[128:] == 3.0).all()
    assert (ca[:k] == 0).all() and (ca[k:] == 3.0).all()
    r2, c2 = O.group_amax_tensor(x, splits, rowwise=False)
    assert r2 is None and np.array_equal(c2, ca)


@pytest.mark.parametrize("seed", range(4))
def test_closed_form_roundtrip_with_one_scale_per_expert(seed):
    """Each expert's values are g * S * 2^j with one 2^j per expert, S a power
    of two constant on each aligned 16 x 16 square (so every rowwise and
    every columnwise block lies in one square), a +-6 on each square's
    diagonal (so every block's amax is 6 * S * 2^j) and one square per
    expert at S = 448: the expert's tensor amax is 2688 * 2^j, every line's
    scale is exactly 2^j and every block's scale is its S, so the plain cast
    reproduces every value in both directions, and so does the four-over-six
    cast with bound 448 (its k = 6 candidate is then exact, error 0)."""
    rng = np.random.default_rng(seed)
    splits, k = [128, 256], 64
    blocks = []
    for m in splits:
        j = int(rng.integers(-20, 20))
        S = 2.0 ** rng.integers(-6, 8, (m // 16, k // 16)).astype(np.float64)
        S[int(rng.integers(0, m // 16)), int(rng.integers(0, k // 16))] = 448.0
        g = GRID[rng.integers(0, 8, (m, k))] * rng.choice([-1.0, 1.0], (m, k))
        r, c = np.meshgrid(np.arange(m), np.arange(k), indexing="ij")
        diag = (r % 16) == (c % 16)
        g[diag] = 6.0 * rng.choice([-1.0, 1.0], int(diag.sum()))
        v = g * np.kron(S, np.ones((16, 16))) * 2.0 ** j
        blocks.append(v)
    xf = np.concatenate(blocks).astype(np.float32)
    x = synth.f32_to_bf16_bits(xf)
    assert np.array_equal(synth.bf16_bits_to_f32(x), xf)
    r = O.group_quantize(x, splits, row_scaled=False)
    assert np.array_equal(O.decode_rowwise(r["row_data"], r["row_scale"], r["row_amax"]), xf)
    assert np.array_equal(O.decode_columnwise(r["col_data"], r["col_scale"], r["col_amax"], splits, k), xf)
    r4 = O.group_quantize_4o6(x, splits, 448, O.ERR_MSE, row_scaled=False)
    assert np.array_equal(r4["row_data"], r["row_data"]) and np.array_equal(r4["row_scale"], r["row_scale"])
    assert np.array_equal(r4["col_data"], r["col_data"]) and np.array_equal(r4["col_scale"], r["col_scale"])


@pytest.mark.parametrize("where", ["first", "last", "middle"])
def test_maximum_at_the_edges_of_an_expert(where):
    """The expert's largest magnitude placed at its first row and column,
    its last row and column, or inside: the tensor amax finds it wherever
    it is (a skipped row or column would miss it)."""
    splits, k = [128, 256, 128], 48
    rng = np.random.default_rng(7)
    xf = rng.standard_normal((512, k)).astype(np.float32)
    offs = np.concatenate([[0], np.cumsum(splits)]).astype(int)
    want = []
    for e in range(len(splits)):
        lo, hi = offs[e], offs[e + 1]
        r, c = {"first": (lo, 0), "last": (hi - 1, k - 1), "middle": ((lo + hi) // 2, k // 2)}[where]
        xf[r, c] = np.float32(-(100.0 + e))
        want.append(np.float32(100.0 + e))
    x = synth.f32_to_bf16_bits(xf)
    ra, ca = O.group_amax_tensor(x, splits)
    for e in range(len(splits)):
        assert (ca[e * k:(e + 1) * k] == want[e]).all()
        assert (ra[offs[e]:offs[e + 1]] == want[e]).all()
