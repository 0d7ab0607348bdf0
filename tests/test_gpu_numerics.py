"""Exhaustive and sampled checks of the device numerics on the GPU.

The kernels quantise with gfx950's hardware FP4 convert and with a block
step whose fast path replaces three correctly rounded divisions by fused
corrections.  These tests prove both equal to their plain definitions on
every input they can receive, and pin GPU outputs to the CPU oracle:

* hardware FP4 convert == the software E2M1 rule, on all 2^32 - 2^24 non-NaN
  fp32 patterns, in both nibble positions;
* hardware E4M3 encode (clamped at 448) == the plain E4M3FN rule on every fp32
  t in [0, +inf], and hardware decode == the rule on every finite code;
* the kernels' block step == the IEEE-division block step, on every pair of
  bf16 values b <= A (532,701,119 pairs: every block amax / line amax pair a
  bf16 input can produce);
* GPU block steps and FP4 codes == the oracle on large structured samples.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

from gpu_helpers import log

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "hip", "libnvfp4g_selftest.so")
P = ctypes.c_void_p


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run tests/hip/build_selftest.py")
    L = ctypes.CDLL(LIB)
    L.selftest_fp4_exhaustive.argtypes = [P]
    L.selftest_block_step_exhaustive.argtypes = [P]
    L.selftest_e4m3_exhaustive.argtypes = [P]
    L.selftest_block_step_sample.argtypes = [P, P, ctypes.c_int64, P, P]
    L.selftest_fp4_codes.argtypes = [P, ctypes.c_int64, P]
    L.selftest_fp4_decode.argtypes = [P]
    L.selftest_rcp_exhaustive.argtypes = [P]
    L.selftest_div6_exhaustive.argtypes = [P]
    L.selftest_quot_4o6_exhaustive.argtypes = [P]
    return L


def ptr(t):
    return P(t.data_ptr())


def test_fp4_convert_equals_software_rule_on_every_fp32(lib):
    log("fp4 convert, all fp32 patterns")
    c = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    assert lib.selftest_fp4_exhaustive(ptr(c)) == 0
    n, bad_lo, bad_hi = c.cpu().tolist()
    assert n == (1 << 32) - 2 * ((1 << 23) - 1)  # all but the NaN patterns
    assert bad_lo == 0 and bad_hi == 0


def test_e4m3_convert_equals_plain_rule_on_every_fp32(lib):
    log("e4m3 convert, all non-negative fp32 patterns")
    c = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    assert lib.selftest_e4m3_exhaustive(ptr(c)) == 0
    n, bad_enc, bad_dec = c.cpu().tolist()
    assert n == 0x7F800001  # +0 .. +inf
    assert bad_enc == 0 and bad_dec == 0


def test_block_step_equals_ieee_divisions_on_every_bf16_pair(lib):
    log("block step, all bf16 pairs b <= A")
    c = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    assert lib.selftest_block_step_exhaustive(ptr(c)) == 0
    n, bad_s, bad_m = c.cpu().tolist()
    amax16 = np.arange(1, 0x7F80, dtype=np.int64)
    assert n == int((amax16 + 1).sum())
    assert bad_s == 0 and bad_m == 0


def _pairs(rng, n):
    """bf16 patterns b <= A: uniform over the finite range, plus line amax near
    the fast path's threshold, tiny and subnormal lines, b = A and b = 0."""
    A = rng.integers(1, 0x7F80, n).astype(np.uint16)
    A[: n // 8] = rng.integers(0x0A00, 0x0E00, n // 8)      # A around 2^-107 .. 2^-99
    A[n // 8: n // 4] = rng.integers(1, 0x0100, n // 8)      # bf16 subnormal / tiny lines
    b = (rng.random(n) * (A.astype(np.float64) + 1)).astype(np.uint16)
    b = np.minimum(b, A)
    b[: 64] = A[: 64]
    b[64: 128] = 0
    return b, A


def test_block_step_sample_matches_oracle(lib):
    rng = np.random.default_rng(3)
    b, A = _pairs(rng, 1 << 20)
    log("block step sample vs oracle")
    db = torch.from_numpy(b.view(np.int16)).cuda()
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    S = torch.empty(b.size, dtype=torch.uint8, device="cuda:0")
    m = torch.empty(b.size, dtype=torch.float32, device="cuda:0")
    assert lib.selftest_block_step_sample(ptr(db), ptr(dA), b.size, ptr(S), ptr(m)) == 0
    torch.cuda.synchronize()
    bf = (b.astype(np.uint32) << 16).view(np.float32)
    Af = (A.astype(np.uint32) << 16).view(np.float32)
    s = (Af / np.float32(2688.0)).astype(np.float32)            # IEEE fp32 division
    rS, rm = O.block_scale(bf, s)
    assert (S.cpu().numpy() == rS).all()
    assert (m.cpu().numpy().view(np.uint32) == rm.view(np.uint32)).all()


def test_fp4_codes_match_oracle(lib):
    # every 37th fp32 pattern up to 8.0, the E2M1 midpoints and their
    # neighbours, denormals, large values, infinities and both zeros, with
    # both signs
    bits = np.arange(0, 0x41000000, 37, dtype=np.uint32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
                            np.array([0.0, 1e-45, 1e-40, 6.0, 6.5, 1e30, np.inf], np.float32)])
    v = np.concatenate([bits.view(np.float32), extra])
    v = np.concatenate([v, -v])
    log(f"fp4 codes vs oracle, {v.size} values")
    dv = torch.from_numpy(v).cuda()
    codes = torch.empty(v.size, dtype=torch.uint8, device="cuda:0")
    assert lib.selftest_fp4_codes(ptr(dv), v.size, ptr(codes)) == 0
    torch.cuda.synchronize()
    assert (codes.cpu().numpy() == O.e2m1_encode(v)).all()


def test_fp4_decode_equals_e2m1_values(lib):
    """The four-over-six cast dequantises each candidate's codes with the
    hardware FP4 -> fp32 convert at unit scale: on every byte, at every byte
    position of the word, both nibbles decode to the E2M1 value of the
    oracle (zero codes compare equal whatever the sign of the zero)."""
    log("fp4 decode, 256 bytes x 4 positions")
    out = torch.empty(2048, dtype=torch.float32, device="cuda:0")
    assert lib.selftest_fp4_decode(ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(256, 4, 2)
    val = np.array([O.e2m1_value(c) for c in range(16)], dtype=np.float32)
    for byte in range(256):
        for sel in range(4):
            assert got[byte, sel, 0] == val[byte & 15], (byte, sel)
            assert got[byte, sel, 1] == val[byte >> 4], (byte, sel)


def test_fast_reciprocal_equals_ieee_on_every_normal_d(lib):
    """rcp_rn (hardware reciprocal + one Newton step) gives the IEEE 1/d on
    every fp32 d in [2^-126, 2^126): the four-over-six cast uses it for the
    element multiplier when its block's d lies in that range."""
    log("fast reciprocal vs IEEE division, 2^31 - 2^24 - ... values")
    c = torch.zeros(2, dtype=torch.int64, device="cuda:0")
    assert lib.selftest_rcp_exhaustive(ptr(c)) == 0
    torch.cuda.synchronize()
    n, bad = c.tolist()
    assert n == 0x7E800000 - 0x00800000
    assert bad == 0, f"{bad} mismatches"


def test_fast_div6_equals_ieee_on_every_bf16(lib):
    """div6_bf16 gives the IEEE b/6 on every finite non-negative bf16 b
    (subnormals and zero included)."""
    c = torch.zeros(2, dtype=torch.int64, device="cuda:0")
    assert lib.selftest_div6_exhaustive(ptr(c)) == 0
    torch.cuda.synchronize()
    n, bad = c.tolist()
    assert n == 0x7F80
    assert bad == 0, f"{bad} mismatches"


def test_fast_quotient_gives_the_ieee_e4m3_code_on_every_4o6_input(lib):
    """quot_fast (u * RN(1/s) plus one residual correction) against the IEEE
    quotient u / s over every input of the four-over-six block step: every
    bf16 line amax A and bound 1..448 with s = A / (6 * bound) >= 2^-112,
    every bf16 block amax b <= A, both candidates (u = b/6, b/4).  The E4M3
    code it yields must always be the IEEE quotient's (the bits may differ
    where both round to the same code)."""
    log("fast quotient vs IEEE division over (A, bound, b, candidate)")
    c = torch.zeros(4, dtype=torch.int64, device="cuda:0")
    assert lib.selftest_quot_4o6_exhaustive(ptr(c)) == 0
    torch.cuda.synchronize()
    n, badt, badS, skipped = c.tolist()
    log(f"{n} quotients, {badt} differ in bits, {badS} in E4M3 code; {skipped} (A, bound) lines skipped")
    assert n > 4 * 10 ** 11
    assert badS == 0
