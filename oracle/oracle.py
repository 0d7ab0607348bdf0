"""Python access to the C oracle (``nvfp4_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product package.  The
oracle shares no code with the HIP library; see the header of
``nvfp4_oracle.c`` for what it computes and which page passages it follows.
The row-scaled grouped GEMM at the end of this file (the cast's consumer) is
plain numpy in float64 on top of the C oracle's two value tables; it is
pinned by ``tests/test_oracle_gemm_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")

# -ffp-contract=off: no FMA contraction, so each float expression in the C
# source is one IEEE binary32 operation; no -ffast-math, no -march=native.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def build() -> str:
    """Compile the oracle with gcc into ``oracle/libnvfp4_oracle.so``."""
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
    os.replace(tmp, LIB)
    return LIB


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it only if it is not built yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [_F]
        L.oracle_e4m3_encode.restype = ctypes.c_int
        L.oracle_e2m1_encode.argtypes = [_F]
        L.oracle_e2m1_encode.restype = ctypes.c_int
        L.oracle_line_scale.argtypes = [_F]
        L.oracle_line_scale.restype = _F
        L.oracle_block_scale.argtypes = [_F, _F, ctypes.POINTER(_F)]
        L.oracle_block_scale.restype = ctypes.c_int
        L.oracle_encode_line.argtypes = [_P, _I64, _F, _P, _P]
        L.oracle_decode_line.argtypes = [_P, _P, _I64, _F, _P]
        L.oracle_row_amax.argtypes = [_P, _I64, _I64]
        L.oracle_row_amax.restype = _F
        L.oracle_col_amax.argtypes = [_P, _I64, _I64, _I64, _I64]
        L.oracle_col_amax.restype = _F
        L.oracle_group_amax.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P]
        L.oracle_group_amax_tensor.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P]
        L.oracle_cast_row.argtypes = [_P, _I64, _I64, _F, _P, _P]
        L.oracle_cast_col.argtypes = [_P, _I64, _I64, _I64, _I64, _F, _P, _P]
        L.oracle_group_cast.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.oracle_e4m3_encode_array.argtypes = [_P, _I64, _P]
        L.oracle_e2m1_encode_array.argtypes = [_P, _I64, _P]
        L.oracle_block_scale_array.argtypes = [_P, _P, _I64, _P, _P]
        L.oracle_mx_scale_byte.argtypes = [_F]
        L.oracle_mx_scale_byte.restype = ctypes.c_int
        L.oracle_mx_encode_line.argtypes = [_P, _I64, _P, _P]
        L.oracle_mx_decode_line.argtypes = [_P, _P, _I64, _P]
        L.oracle_mxfp4_group_cast.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P]
        L.oracle_mx_scale_byte_array.argtypes = [_P, _I64, _P]
        L.oracle_line_scale_b.argtypes = [_F, ctypes.c_int]
        L.oracle_line_scale_b.restype = _F
        L.oracle_block_4o6.argtypes = [_P, _F, ctypes.c_int, _P, _P, _P]
        L.oracle_block_4o6.restype = ctypes.c_int
        L.oracle_encode_line_4o6.argtypes = [_P, _I64, _F, ctypes.c_int, ctypes.c_int, _P, _P, _P]
        L.oracle_decode_line_b.argtypes = [_P, _P, _I64, _F, ctypes.c_int, _P]
        L.oracle_group_cast_4o6.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                            _P, _P, _P, _P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


# --------------------------------------------------------------- conversions

def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.int32)
    lib().oracle_e4m3_encode_array(_ptr(t), t.size, _ptr(out))
    return out


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.int32)
    lib().oracle_e2m1_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def line_scale(amax: float) -> np.float32:
    return np.float32(lib().oracle_line_scale(float(amax)))


def block_scale(b: np.ndarray, s: np.ndarray):
    """Vector form of the block step: returns (E4M3 codes, multipliers m)."""
    b = np.ascontiguousarray(b, dtype=np.float32)
    s = np.ascontiguousarray(np.broadcast_to(s, b.shape), dtype=np.float32)
    S = np.empty(b.shape, dtype=np.int32)
    m = np.empty(b.shape, dtype=np.float32)
    lib().oracle_block_scale_array(_ptr(b), _ptr(s), b.size, _ptr(S), _ptr(m))
    return S, m


# ------------------------------------------------------------------- lines

def encode_line(L: np.ndarray, amax: float):
    L = np.ascontiguousarray(L, dtype=np.float32)
    n = L.size
    codes = np.empty(n // 2, dtype=np.uint8)
    scales = np.empty(n // 16, dtype=np.uint8)
    _check(lib().oracle_encode_line(_ptr(L), n, float(amax), _ptr(codes), _ptr(scales)), "encode_line")
    return codes, scales


def decode_line(codes: np.ndarray, scales: np.ndarray, n: int, amax: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty(n, dtype=np.float32)
    _check(lib().oracle_decode_line(_ptr(codes), _ptr(scales), n, float(amax), _ptr(out)), "decode_line")
    return out


def row_amax(x: np.ndarray, r: int) -> np.float32:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return np.float32(lib().oracle_row_amax(_ptr(x), x.shape[1], int(r)))


def col_amax(x: np.ndarray, c: int, r0: int, m: int) -> np.float32:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return np.float32(lib().oracle_col_amax(_ptr(x), x.shape[1], int(c), int(r0), int(m)))


def cast_row(x: np.ndarray, r: int, amax: float):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    k = x.shape[1]
    data = np.empty(k // 2, dtype=np.uint8)
    sc = np.empty(k // 16, dtype=np.uint8)
    _check(lib().oracle_cast_row(_ptr(x), k, int(r), float(amax), _ptr(data), _ptr(sc)), "cast_row")
    return data, sc


def cast_col(x: np.ndarray, c: int, r0: int, m: int, amax: float):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    k = x.shape[1]
    data = np.empty(m // 2, dtype=np.uint8)
    sc = np.empty(m // 16, dtype=np.uint8)
    _check(lib().oracle_cast_col(_ptr(x), k, int(c), int(r0), int(m), float(amax), _ptr(data), _ptr(sc)),
           "cast_col")
    return data, sc


# ---------------------------------------------------------------- grouped

def group_amax(x: np.ndarray, splits, rowwise: bool = True, columnwise: bool = True):
    """Grouped amax over packed bf16 bits ``x`` (sum_m, k) with host splits."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sum_m, k = x.shape
    sp = np.ascontiguousarray(splits, dtype=np.int64)
    E = sp.size
    ra = np.empty(sum_m, dtype=np.float32) if rowwise else None
    ca = np.empty(E * k, dtype=np.float32) if columnwise else None
    _check(lib().oracle_group_amax(_ptr(x), sum_m, k, E, _ptr(sp), _ptr(ra), _ptr(ca)), "group_amax")
    return ra, ca


def group_amax_tensor(x: np.ndarray, splits, rowwise: bool = True, columnwise: bool = True):
    """Per-tensor amax (row scaling off): every line of expert e gets the
    expert's max |x|; returned as the (row_amax, col_amax) vectors."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sum_m, k = x.shape
    sp = np.ascontiguousarray(splits, dtype=np.int64)
    E = sp.size
    ra = np.empty(sum_m, dtype=np.float32) if rowwise else None
    ca = np.empty(E * k, dtype=np.float32) if columnwise else None
    _check(lib().oracle_group_amax_tensor(_ptr(x), sum_m, k, E, _ptr(sp), _ptr(ra), _ptr(ca)), "group_amax_tensor")
    return ra, ca


def group_cast(x: np.ndarray, splits, row_amax=None, col_amax=None,
               rowwise: bool = True, columnwise: bool = True):
    """Grouped cast.  Returns (row_data, row_scale, col_data, col_scale); the
    arrays of a direction not requested are None."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sum_m, k = x.shape
    sp = np.ascontiguousarray(splits, dtype=np.int64)
    E = sp.size
    rd = np.empty((sum_m, k // 2), dtype=np.uint8) if rowwise else None
    rs = np.empty((sum_m, k // 16), dtype=np.uint8) if rowwise else None
    cd = np.empty(sum_m * k // 2, dtype=np.uint8) if columnwise else None
    cs = np.empty(sum_m * k // 16, dtype=np.uint8) if columnwise else None
    ra = None if row_amax is None else np.ascontiguousarray(row_amax, dtype=np.float32)
    ca = None if col_amax is None else np.ascontiguousarray(col_amax, dtype=np.float32)
    _check(lib().oracle_group_cast(_ptr(x), sum_m, k, E, _ptr(sp), _ptr(ra), _ptr(ca),
                                   _ptr(rd), _ptr(rs), _ptr(cd), _ptr(cs)), "group_cast")
    return rd, rs, cd, cs


def group_quantize(x: np.ndarray, splits, rowwise: bool = True, columnwise: bool = True, row_scaled: bool = True):
    """Amax (per line, or per expert tensor when row_scaled is False) then
    cast, as one dict of numpy arrays."""
    ra, ca = (group_amax if row_scaled else group_amax_tensor)(x, splits, rowwise, columnwise)
    rd, rs, cd, cs = group_cast(x, splits, ra, ca, rowwise, columnwise)
    return {"row_amax": ra, "col_amax": ca, "row_data": rd, "row_scale": rs,
            "col_data": cd, "col_scale": cs}


def decode_rowwise(row_data, row_scale, row_amax) -> np.ndarray:
    """Dequantize the whole rowwise output to fp32 (sum_m, k)."""
    sum_m = row_data.shape[0]
    k = row_data.shape[1] * 2
    out = np.empty((sum_m, k), dtype=np.float32)
    for r in range(sum_m):
        out[r] = decode_line(row_data[r], row_scale[r], k, row_amax[r])
    return out


def decode_columnwise(col_data, col_scale, col_amax, splits, k: int):
    """Dequantize the columnwise output back to the (sum_m, k) layout."""
    sp = [int(v) for v in splits]
    sum_m = sum(sp)
    out = np.empty((sum_m, k), dtype=np.float32)
    r0 = 0
    for e, m in enumerate(sp):
        d = col_data[k * r0 // 2: k * (r0 + m) // 2].reshape(k, m // 2) if m else None
        s = col_scale[k * r0 // 16: k * (r0 + m) // 16].reshape(k, m // 16) if m else None
        for c in range(k if m else 0):
            out[r0:r0 + m, c] = decode_line(d[c], s[c], m, col_amax[e * k + c])
        r0 += m
    return out


# ------------------------------------------------------------------ MXFP4

def mx_scale_byte(A: np.ndarray) -> np.ndarray:
    A = np.ascontiguousarray(A, dtype=np.float32)
    out = np.empty(A.shape, dtype=np.int32)
    lib().oracle_mx_scale_byte_array(_ptr(A), A.size, _ptr(out))
    return out


def mx_encode_line(L: np.ndarray):
    L = np.ascontiguousarray(L, dtype=np.float32)
    n = L.size
    codes = np.empty(n // 2, dtype=np.uint8)
    scales = np.empty(n // 32, dtype=np.uint8)
    _check(lib().oracle_mx_encode_line(_ptr(L), n, _ptr(codes), _ptr(scales)), "mx_encode_line")
    return codes, scales


def mx_decode_line(codes, scales, n: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty(n, dtype=np.float32)
    _check(lib().oracle_mx_decode_line(_ptr(codes), _ptr(scales), n, _ptr(out)), "mx_decode_line")
    return out


def mxfp4_group_cast(x: np.ndarray, splits, rowwise: bool = True, columnwise: bool = True):
    """Grouped MXFP4 cast: (row_data, row_scale, col_data, col_scale)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sum_m, k = x.shape
    sp = np.ascontiguousarray(splits, dtype=np.int64)
    rd = np.empty((sum_m, k // 2), dtype=np.uint8) if rowwise else None
    rs = np.empty((sum_m, k // 32), dtype=np.uint8) if rowwise else None
    cd = np.empty(sum_m * k // 2, dtype=np.uint8) if columnwise else None
    cs = np.empty(sum_m * k // 32, dtype=np.uint8) if columnwise else None
    _check(lib().oracle_mxfp4_group_cast(_ptr(x), sum_m, k, sp.size, _ptr(sp), _ptr(rd), _ptr(rs), _ptr(cd),
                                         _ptr(cs)), "mxfp4_group_cast")
    return rd, rs, cd, cs


# ---------------------------------------------------------- four over six
#
# The four-over-six block scaling of nvfp4_oracle.c (each block encoded with
# its amax mapped to 6 and to 4, the smaller error kept; line scale
# A / (6 * bound)).

DEFAULT_4O6_BOUND = 256
ERR_MSE, ERR_MAE = 0, 1


def line_scale_b(amax: float, bound: int) -> np.float32:
    return np.float32(lib().oracle_line_scale_b(float(amax), int(bound)))


def block_4o6(blk, s: float, err_mode: int = ERR_MSE):
    """One 16-element block: (E4M3 code, 16 codes, pick 4 or 6, (err_6, err_4))."""
    blk = np.ascontiguousarray(blk, dtype=np.float32)
    assert blk.size == 16
    codes = np.empty(16, dtype=np.int32)
    pick = ctypes.c_int()
    errs = np.empty(2, dtype=np.float32)
    S = lib().oracle_block_4o6(_ptr(blk), float(s), int(err_mode), _ptr(codes), ctypes.byref(pick), _ptr(errs))
    return S, codes, pick.value, (errs[0], errs[1])


def encode_line_4o6(L, amax: float, bound: int = DEFAULT_4O6_BOUND, err_mode: int = ERR_MSE):
    """(packed codes, E4M3 scales, picks) of one line."""
    L = np.ascontiguousarray(L, dtype=np.float32)
    n = L.size
    codes = np.empty(n // 2, dtype=np.uint8)
    scales = np.empty(n // 16, dtype=np.uint8)
    picks = np.empty(n // 16, dtype=np.uint8)
    _check(lib().oracle_encode_line_4o6(_ptr(L), n, float(amax), int(bound), int(err_mode), _ptr(codes),
                                        _ptr(scales), _ptr(picks)), "encode_line_4o6")
    return codes, scales, picks


def decode_line_b(codes, scales, n: int, amax: float, bound: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty(n, dtype=np.float32)
    _check(lib().oracle_decode_line_b(_ptr(codes), _ptr(scales), n, float(amax), int(bound), _ptr(out)),
           "decode_line_b")
    return out


def group_cast_4o6(x: np.ndarray, splits, row_amax=None, col_amax=None, bound: int = DEFAULT_4O6_BOUND,
                   err_mode: int = ERR_MSE, rowwise: bool = True, columnwise: bool = True):
    """Grouped four-over-six cast: (row_data, row_scale, col_data, col_scale)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sum_m, k = x.shape
    sp = np.ascontiguousarray(splits, dtype=np.int64)
    rd = np.empty((sum_m, k // 2), dtype=np.uint8) if rowwise else None
    rs = np.empty((sum_m, k // 16), dtype=np.uint8) if rowwise else None
    cd = np.empty(sum_m * k // 2, dtype=np.uint8) if columnwise else None
    cs = np.empty(sum_m * k // 16, dtype=np.uint8) if columnwise else None
    ra = None if row_amax is None else np.ascontiguousarray(row_amax, dtype=np.float32)
    ca = None if col_amax is None else np.ascontiguousarray(col_amax, dtype=np.float32)
    _check(lib().oracle_group_cast_4o6(_ptr(x), sum_m, k, sp.size, _ptr(sp), _ptr(ra), _ptr(ca), int(bound),
                                       int(err_mode), _ptr(rd), _ptr(rs), _ptr(cd), _ptr(cs)), "group_cast_4o6")
    return rd, rs, cd, cs


def group_quantize_4o6(x: np.ndarray, splits, bound: int = DEFAULT_4O6_BOUND, err_mode: int = ERR_MSE,
                       rowwise: bool = True, columnwise: bool = True, row_scaled: bool = True):
    """Amax (per line, or per expert tensor when row_scaled is False) then
    the four-over-six cast."""
    ra, ca = (group_amax if row_scaled else group_amax_tensor)(x, splits, rowwise, columnwise)
    rd, rs, cd, cs = group_cast_4o6(x, splits, ra, ca, bound, err_mode, rowwise, columnwise)
    return {"row_amax": ra, "col_amax": ca, "row_data": rd, "row_scale": rs, "col_data": cd, "col_scale": cs}


# ------------------------------------------------- row-scaled grouped GEMM
#
# The consumer of the cast ("Implement per-token NVFP4 fprop recipe",
# TransformerEngine PR 2931, Greptile Summary and its sequence diagram: the
# GEMM runs on the block-scaled FP4 operands with the row amax set aside, and
# its fp32 output rows are then multiplied by the row amax; "[PyTorch] Enable
# NVFP4 row-scaled (per-token) backward for GroupedLinear", TransformerEngine
# PR 3324, Greptile Summary: the NT weight-gradient GEMM runs per expert on
# the columnwise operands).  Here each operand element is dequantised in exact
# arithmetic,  x = value(code) * value(S) * (A / 2688),  and the GEMM is the
# plain product of the dequantised matrices.  It is evaluated in float64:
# value(code) * value(S) is exact there, and a float64 dot product of
# thousands of such terms is far more accurate than the fp32 result under
# test.  The second return value is the same product taken over absolute
# values, the scale of the rounding-error bound of an fp32 evaluation.

def _values_table():
    q = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    s = np.array([e4m3_value(c) if c != 0x7F else np.nan for c in range(256)], dtype=np.float64)
    return q, s


def block_values(data: np.ndarray, scale: np.ndarray, n: int) -> np.ndarray:
    """value(code) * value(S) for every element of `rows` lines of n elements:
    data [rows, n/2] (element 2j in the low nibble of byte j), scale
    [rows, n/16] E4M3 codes.  Exact in float64."""
    q, s = _values_table()
    data = np.asarray(data, dtype=np.uint8).reshape(-1, n // 2)
    scale = np.asarray(scale, dtype=np.uint8).reshape(-1, n // 16)
    codes = np.empty((data.shape[0], n), dtype=np.uint8)
    codes[:, 0::2] = data & 15
    codes[:, 1::2] = data >> 4
    return q[codes] * np.repeat(s[scale], 16, axis=1)


def _line_scales(amax) -> np.ndarray:
    return np.asarray(amax, dtype=np.float32).astype(np.float64) / 2688.0


def group_gemm(a_data, a_scale, a_amax, b_data, b_scale, b_amax, splits, n: int, k: int):
    """Grouped row-scaled GEMM, forward form.  For expert e with rows
    [r_e, r_e + M_e) of a:  out[r, j] = sum_t xa[r, t] * xb_e[j, t]  with
    a = (a_data [sum_m, k/2], a_scale [sum_m, k/16], a_amax [sum_m]) and
    b_e = (b_data [E, n, k/2], b_scale [E, n, k/16], b_amax [E*n]) row-scaled
    NVFP4 operands.  Returns (out, bound_scale), both float64 [sum_m, n]."""
    sp = [int(v) for v in splits]
    sum_m = sum(sp)
    E = len(sp)
    a_vals = block_values(a_data, a_scale, k) if sum_m else np.zeros((0, k))
    sa = _line_scales(a_amax)
    b_vals = block_values(b_data, b_scale, k).reshape(E, n, k)
    sb = _line_scales(b_amax).reshape(E, n)
    out = np.zeros((sum_m, n), dtype=np.float64)
    bound = np.zeros((sum_m, n), dtype=np.float64)
    r0 = 0
    for e, m in enumerate(sp):
        if m:
            A = a_vals[r0:r0 + m]
            B = b_vals[e]
            scale = np.outer(sa[r0:r0 + m], sb[e])
            out[r0:r0 + m] = (A @ B.T) * scale
            bound[r0:r0 + m] = (np.abs(A) @ np.abs(B).T) * np.abs(scale)
        r0 += m
    return out, bound


def group_gemm_wgrad(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax,
                     splits, n: int, k: int):
    """Grouped row-scaled GEMM, weight-gradient form, on two columnwise
    (transposed) cast outputs: a = dY's ([n, M_e] lines of expert e at byte
    n*r_e/2, amax a_col_amax[e*n + i]) and b = X's ([k, M_e] lines, amax
    b_col_amax[e*k + j]).  out[e, i, j] = sum_{t < M_e} xa_e[i, t] * xb_e[j, t],
    i.e. dW_e = dY_e^T X_e; an expert without rows gets zeros.  Returns
    (out, bound_scale), float64 [E, n, k]."""
    sp = [int(v) for v in splits]
    E = len(sp)
    sa = _line_scales(a_col_amax).reshape(E, n)
    sb = _line_scales(b_col_amax).reshape(E, k)
    out = np.zeros((E, n, k), dtype=np.float64)
    bound = np.zeros((E, n, k), dtype=np.float64)
    r0 = 0
    for e, m in enumerate(sp):
        if m:
            A = block_values(a_col_data[n * r0 // 2: n * (r0 + m) // 2], a_col_scale[n * r0 // 16: n * (r0 + m) // 16], m)
            B = block_values(b_col_data[k * r0 // 2: k * (r0 + m) // 2], b_col_scale[k * r0 // 16: k * (r0 + m) // 16], m)
            scale = np.outer(sa[e], sb[e])
            out[e] = (A @ B.T) * scale
            bound[e] = (np.abs(A) @ np.abs(B).T) * np.abs(scale)
        r0 += m
    return out, bound
