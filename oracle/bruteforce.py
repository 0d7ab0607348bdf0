"""Independent brute-force re-statement of the row-scaled NVFP4 cast.

TEST INFRASTRUCTURE ONLY (imported by ``tests/``).  It shares nothing with
either the C oracle or the HIP library: conversions are done by exhaustive
nearest-value search over every code of the target format, written with numpy
float32 (IEEE binary32, round-to-nearest-even) for each arithmetic step of the
fixed reading:

    s = A / (6*448);  t = (b/6)/s;  S = E4M3(t);  d = value(S)*s;
    m = 1/d (0 if d == 0, clamped to FLT_MAX);  code = E2M1(x*m)

(per-token NVFP4 from "Implement per-token NVFP4 fprop recipe", Description;
grouped amax and cast from the TransformerEngine issue 3649 page
(single-launch grouped row-scaled NVFP4 cast), Description).  Meant for tiny inputs: it is vectorised over elements
but tries all 16 (or 127) candidates for each one.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
FLT_MAX = np.finfo(np.float32).max


def _e4m3_table() -> np.ndarray:
    """All 127 non-negative finite E4M3FN values, by code (0x00..0x7E)."""
    vals = []
    for code in range(0x7F):
        e, f = code >> 3, code & 7
        vals.append(f * 2.0 ** -9 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3 = _e4m3_table()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _nearest_even(table: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Index of the nearest table entry for each a (float64-exact distances);
    among equally near entries the even index wins; beyond the last entry the
    last index (saturation)."""
    a = np.asarray(a, dtype=np.float64)
    dist = np.abs(a[..., None] - table)                   # exact in float64
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    idx = np.arange(table.size)
    # prefer even indices among ties, then the smaller one
    score = np.where(cand, (idx % 2) * table.size + idx, 10 * table.size)
    out = score.argmin(axis=-1)
    return np.where(a >= table[-1], table.size - 1, out)


def e4m3_encode(t) -> np.ndarray:
    return _nearest_even(E4M3, t)


def e2m1_encode(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32)
    mag = _nearest_even(E2M1, np.abs(v).astype(np.float64))
    return mag | (np.signbit(v).astype(np.int64) << 3)


def encode_line(L, A):
    """Encode a line (float32, length a multiple of 16) with line amax A.
    Returns (packed bytes, E4M3 codes)."""
    L = np.asarray(L, dtype=np.float32)
    n = L.size
    s = F32(A) / (F32(6.0) * F32(448.0))
    blocks = L.reshape(n // 16, 16)
    b = np.abs(blocks).max(axis=1).astype(np.float32) if n else np.zeros(0, np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        t = np.where(s == F32(0), F32(0), (b / F32(6.0)) / s).astype(np.float32)
        S = e4m3_encode(t)
        d = E4M3[S].astype(np.float32) * s
        m = np.where(d == F32(0), F32(0), np.minimum(F32(1.0) / d, FLT_MAX)).astype(np.float32)
        v = (blocks * m[:, None]).astype(np.float32)
    codes = e2m1_encode(v).reshape(-1)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, S.astype(np.uint8)


def bf16_to_f32(x_bits: np.ndarray) -> np.ndarray:
    return (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def group_quantize(x_bits, splits, rowwise=True, columnwise=True):
    """Brute-force grouped amax + cast; same output layout as the C oracle."""
    x = bf16_to_f32(x_bits)
    sum_m, k = x.shape
    splits = [int(v) for v in splits]
    out = {}
    if rowwise:
        ra = np.abs(x).max(axis=1).astype(np.float32) if k else np.zeros(sum_m, np.float32)
        rd = np.empty((sum_m, k // 2), np.uint8)
        rs = np.empty((sum_m, k // 16), np.uint8)
        for r in range(sum_m):
            rd[r], rs[r] = encode_line(x[r], ra[r])
        out.update(row_amax=ra, row_data=rd, row_scale=rs)
    if columnwise:
        ca = np.zeros(len(splits) * k, np.float32)
        cd = np.empty(sum_m * k // 2, np.uint8)
        cs = np.empty(sum_m * k // 16, np.uint8)
        r0 = 0
        for e, m in enumerate(splits):
            if m:
                xe = x[r0:r0 + m]
                ca[e * k:(e + 1) * k] = np.abs(xe).max(axis=0)
                for c in range(k):
                    d, s = encode_line(xe[:, c], ca[e * k + c])
                    cd[k * r0 // 2 + c * (m // 2): k * r0 // 2 + (c + 1) * (m // 2)] = d
                    cs[k * r0 // 16 + c * (m // 16): k * r0 // 16 + (c + 1) * (m // 16)] = s
            r0 += m
        out.update(col_amax=ca, col_data=cd, col_scale=cs)
    return out


# ------------------------------------------------------------------ MXFP4

def mx_encode_line(L):
    """MXFP4 (OCP MX v1.0 reading): shared exponent floor(log2(block amax)) - 2
    clamped to [-127, 127] (-127 for an all-zero block), E8M0 byte shared+127,
    codes by nearest-value search over E2M1 of x / 2^shared."""
    L = np.asarray(L, dtype=np.float32)
    blocks = L.reshape(-1, 32).astype(np.float64)
    A = np.abs(blocks).max(axis=1)
    mant, ex = np.frexp(A)                        # A = mant * 2^ex, mant in [0.5, 1)
    shared = np.where(A > 0, ex - 1 - 2, -127)
    shared = np.clip(shared, -127, 127)
    v = blocks / np.ldexp(1.0, shared)[:, None]   # exact in float64
    mag = _nearest_even(E2M1, np.abs(v))
    codes = (mag | (np.signbit(blocks).astype(np.int64) << 3)).reshape(-1)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, (shared + 127).astype(np.uint8)


# ---------------------------------------------------------- four over six

def block_4o6(blk, s, err_mode: int = 0):
    """Four-over-six step of one 16-element block by nearest-value search:
    both candidates (amax mapped to 6, then to 4), each error summed in
    float32 in element order, candidate 4 kept only when its error is
    strictly smaller.  Returns (E4M3 code, 16 codes, pick)."""
    blk = np.asarray(blk, dtype=np.float32)
    s = F32(s)
    b = F32(np.abs(blk).max())
    out = []
    for kk in (F32(6.0), F32(4.0)):
        with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
            t = F32(0) if s == F32(0) else F32(F32(b / kk) / s)
            S = int(e4m3_encode(np.array([t]))[0])
            Sv = F32(E4M3[S])
            d = F32(Sv * s)
            m = F32(0) if d == F32(0) else F32(min(F32(F32(1.0) / d), FLT_MAX))
            codes = e2m1_encode((blk * m).astype(np.float32))
            e = F32(0)
            for i in range(16):
                q = F32(E2M1[codes[i] & 7] * (-1.0 if codes[i] & 8 else 1.0))
                xh = F32(F32(q * Sv) * s)
                diff = F32(blk[i] - xh)
                e = F32(e + (F32(diff * diff) if err_mode == 0 else F32(abs(diff))))
        out.append((S, codes, e))
    (S6, c6, e6), (S4, c4, e4) = out
    return (S4, c4, 4) if e4 < e6 else (S6, c6, 6)


def encode_line_4o6(L, A, bound: int = 256, err_mode: int = 0):
    """(packed bytes, E4M3 codes, picks) of one line, line scale A / (6 * bound)."""
    L = np.asarray(L, dtype=np.float32)
    s = F32(F32(A) / F32(F32(6.0) * F32(bound)))
    S_all, codes_all, picks = [], [], []
    for j in range(L.size // 16):
        S, c, p = block_4o6(L[16 * j:16 * j + 16], s, err_mode)
        S_all.append(S)
        codes_all.append(c)
        picks.append(p)
    codes = np.concatenate(codes_all) if codes_all else np.zeros(0, np.int64)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, np.array(S_all, np.uint8), np.array(picks, np.uint8)
