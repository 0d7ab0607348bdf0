"""Pins of the oracle's MXFP4 cast (the sibling format of the TransformerEngine
PR 3824 page: E2M1 elements, blocks of 32, E8M0 power-of-two scales; scale
rule read from the OCP Microscaling (MX) v1.0 definition) against what the
definition and the mathematics fix.  No GPU."""
import os

import numpy as np
import pytest

from nvfp4_block_scaled_group_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_mx_k64.txt")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_scale_byte_defining_property(O):
    # shared = floor(log2 A) - 2  <=>  4 <= A / 2^shared < 8, within the E8M0 range
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16     # every normal bf16 value
    A = bits.view(np.float32)
    byte = O.mx_scale_byte(A)
    shared = byte.astype(np.int64) - 127
    q = A.astype(np.float64) / np.ldexp(1.0, shared)
    inrange = (shared > -127)
    assert ((q[inrange] >= 4) & (q[inrange] < 8)).all()
    assert (q[~inrange] < 8).all()                     # clamped at the bottom: smaller quotients
    assert O.mx_scale_byte(np.array([0.0], np.float32))[0] == 0
    assert (O.mx_scale_byte((np.arange(1, 0x80, dtype=np.uint32) << 16).view(np.float32)) == 0).all()


def test_closed_form_roundtrip(O):
    # blocks g * 2^j with one element at +-4 or +-6: floor(log2 A) = j + 2, so
    # shared = j and every element is reproduced exactly
    rng = np.random.default_rng(81)
    for _ in range(200):
        nb = int(rng.integers(1, 6))
        L = np.empty(32 * nb, np.float64)
        for b in range(nb):
            j = int(rng.integers(-120, 120))
            g = GRID[rng.integers(0, 8, 32)] * rng.choice([-1.0, 1.0], 32)
            g[rng.integers(0, 32)] = rng.choice([4.0, 6.0]) * rng.choice([-1.0, 1.0])
            L[32 * b: 32 * (b + 1)] = g * 2.0 ** j
        L = L.astype(np.float32)
        codes, scales = O.mx_encode_line(L)
        back = O.mx_decode_line(codes, scales, L.size)
        assert (back.view(np.uint32) == L.view(np.uint32)).all()


def test_saturation_ties_and_zero_block(O):
    L = np.zeros(32, np.float32)
    L[:4] = [7.0, 5.0, -1.25, 0.25]       # A = 7: shared 0; 7 saturates to 6, ties go to even codes
    codes, scales = O.mx_encode_line(L)
    assert scales.tolist() == [127]
    assert codes[:2].tolist() == [7 | (6 << 4), (8 | 2) | (0 << 4)]
    z = np.zeros(32, np.float32)
    z[3] = -0.0
    codes, scales = O.mx_encode_line(z)
    assert scales.tolist() == [0] and codes[1] == 0x80 and (np.delete(codes, 1) == 0).all()


def test_golden_worked_mx(O, BF):
    xs, exp = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            if key == "x":
                xs += [int(v, 16) for v in vals]
            else:
                exp[key] = [int(v, 16) for v in vals]
    L = synth.bf16_bits_to_f32(np.array(xs, np.uint16))
    codes, scales = O.mx_encode_line(L)
    assert codes.tolist() == exp["data"] and scales.tolist() == exp["scale"]
    bc, bs = BF.mx_encode_line(L)
    assert bc.tolist() == exp["data"] and bs.tolist() == exp["scale"]


@pytest.mark.parametrize("seed,splits,k,dist", [
    (82, [128, 0, 256], 64, "normal"), (83, [256], 96, "outliers"), (84, [128, 128], 32, "sparse"),
    (85, [128], 160, "student"), (86, [256, 128], 64, "rowscale"),
])
def test_mx_matches_bruteforce(O, BF, seed, splits, k, dist):
    w = synth.random_case(seed, splits, k, dist)
    rd, rs, cd, cs = O.mxfp4_group_cast(w.x, w.splits)
    xf = synth.bf16_bits_to_f32(w.x)
    for r in range(w.sum_m):
        d, s = BF.mx_encode_line(xf[r])
        assert (rd[r] == d).all() and (rs[r] == s).all()
    r0 = 0
    for m in w.splits:
        m = int(m)
        for c in range(k if m else 0):
            d, s = BF.mx_encode_line(xf[r0:r0 + m, c])
            base = k * r0 + c * m
            assert (cd[base // 2:(base + m) // 2] == d).all()
            assert (cs[base // 32:(base + m) // 32] == s).all()
        r0 += m


def test_mx_grouped_equals_per_expert_and_transpose(O):
    # K = 128 so that an expert's transpose is itself a valid one-expert input
    w = synth.random_case(87, [256, 0, 128, 384], 128, "outliers")
    rd, rs, cd, cs = O.mxfp4_group_cast(w.x, w.splits)
    k, r0 = w.k, 0
    for m in w.splits:
        m = int(m)
        if m:
            a = O.mxfp4_group_cast(w.x[r0:r0 + m], [m])
            assert (a[0] == rd[r0:r0 + m]).all() and (a[1] == rs[r0:r0 + m]).all()
            assert (a[2] == cd[k * r0 // 2:k * (r0 + m) // 2]).all()
            assert (a[3] == cs[k * r0 // 32:k * (r0 + m) // 32]).all()
            # columnwise output of the expert == rowwise output of its transpose
            t = O.mxfp4_group_cast(np.ascontiguousarray(w.x[r0:r0 + m].T), [k], True, False)
            assert (t[0].reshape(-1) == a[2]).all() and (t[1].reshape(-1) == a[3]).all()
        r0 += m


def test_mx_rejects_k_not_multiple_of_32(O):
    with pytest.raises(ValueError):
        O.mxfp4_group_cast(np.zeros((128, 48), np.uint16), [128])
