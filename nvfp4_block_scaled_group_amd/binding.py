"""Thin ctypes binding of ``libnvfp4g.so`` (C ABI in ``include/nvfp4_group.h``).

Each function has the name of the C entry point it calls and only marshals
arguments: torch device tensors become raw pointers, the current HIP stream
is passed along, and a non-zero status raises ``Nvfp4GroupError``.  All work
happens in the library's HIP kernels; if the library is missing, every call
raises (there is no fallback).

Buffers are owned by the caller; ``alloc_outputs`` is a convenience that
allocates them with torch.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4g.so")

NVFP4G_OK = 0
NVFP4G_EINVAL = -1
NVFP4G_ESPLITS = -2
NVFP4G_EALIGN = -3
NVFP4G_EHIP = -4
NVFP4G_DEV_UNALIGNED = 1
NVFP4G_DEV_NONMONO = 2
NVFP4G_DEV_OVERFLOW = 4
MAX_EXPERTS_HOST = 512
MAX_EXPERTS_DEVICE = 4096
# nvfp4_group_quantize{,_graphsafe} with a columnwise output runs as one
# launch when every expert's rows * k <= SMALL_MAX_EXPERT_ELEMS (the
# capacity's for device routing) and k <= SMALL_MAX_K
SMALL_MAX_EXPERT_ELEMS = 1 << 16
SMALL_MAX_K = 512

EXPORTS = (
    "nvfp4_group_amax", "nvfp4_group_cast", "nvfp4_group_amax_graphsafe",
    "nvfp4_group_cast_graphsafe", "nvfp4_group_quantize", "nvfp4_group_quantize_graphsafe",
    "nvfp4_group_dequant_rowwise", "nvfp4_group_dequant_columnwise",
    "nvfp4_group_dequant_columnwise_graphsafe", "mxfp4_group_cast", "mxfp4_group_cast_graphsafe",
    "nvfp4_group_gemm", "nvfp4_group_gemm_graphsafe", "nvfp4_group_gemm_wgrad", "nvfp4_group_gemm_wgrad_graphsafe",
    "nvfp4_group_strerror",
)


class Nvfp4GroupError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None
_P, _I64, _I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (torch is imported first so that the library binds
    to the HIP runtime torch already uses)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m nvfp4_block_scaled_group_amd.build`")
    L = ctypes.CDLL(path)
    L.nvfp4_group_amax.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P]
    L.nvfp4_group_cast.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P]
    L.nvfp4_group_amax_graphsafe.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P]
    L.nvfp4_group_cast_graphsafe.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    L.nvfp4_group_quantize.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P]
    L.nvfp4_group_quantize_graphsafe.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    L.nvfp4_group_dequant_rowwise.argtypes = [_P, _P, _P, _I64, _I64, _P, _P]
    L.nvfp4_group_dequant_columnwise.argtypes = [_P, _P, _P, _I64, _I64, _I32, _P, _P, _P]
    L.nvfp4_group_dequant_columnwise_graphsafe.argtypes = [_P, _P, _P, _I64, _I64, _I32, _P, _P, _P, _P]
    L.mxfp4_group_cast.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P]
    L.mxfp4_group_cast_graphsafe.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
    L.nvfp4_group_gemm.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P]
    L.nvfp4_group_gemm_graphsafe.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P, _P]
    L.nvfp4_group_gemm_wgrad.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P]
    L.nvfp4_group_gemm_wgrad_graphsafe.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P, _P]
    for name in EXPORTS[:-1]:
        getattr(L, name).restype = ctypes.c_int
    L.nvfp4_group_strerror.argtypes = [ctypes.c_int]
    L.nvfp4_group_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(status: int) -> str:
    return load_library().nvfp4_group_strerror(int(status)).decode()


def _check(fn: str, rc: int):
    if rc != NVFP4G_OK:
        raise Nvfp4GroupError(fn, rc, strerror(rc))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _x(x: torch.Tensor):
    if x.dim() != 2 or x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("x must be a 2-D bf16 (or raw 16-bit) tensor")
    return _ptr(x), x.shape[0], x.shape[1]


# the current stream's raw handle without building a Stream object (~0.1 us
# against ~3 us per call for torch.cuda.current_stream())
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        if _raw_current_stream is not None:
            return ctypes.c_void_p(_raw_current_stream(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _splits(h_splits: Sequence[int]):
    arr = (ctypes.c_int64 * len(h_splits))(*[int(v) for v in h_splits])
    return arr, len(h_splits)


# ------------------------------------------------------------ entry points

def nvfp4_group_amax(x, h_splits, row_amax=None, col_amax=None, stream=None):
    xp, m, k = _x(x)
    sp, e = _splits(h_splits)
    _check("nvfp4_group_amax", load_library().nvfp4_group_amax(
        xp, m, k, e, sp, _ptr(row_amax), _ptr(col_amax), _stream(stream)))


def nvfp4_group_cast(x, h_splits, row_amax=None, col_amax=None, row_data=None, row_scale=None,
                     col_data=None, col_scale=None, stream=None):
    xp, m, k = _x(x)
    sp, e = _splits(h_splits)
    _check("nvfp4_group_cast", load_library().nvfp4_group_cast(
        xp, m, k, e, sp, _ptr(row_amax), _ptr(col_amax), _ptr(row_data), _ptr(row_scale),
        _ptr(col_data), _ptr(col_scale), _stream(stream)))


def nvfp4_group_quantize(x, h_splits, row_amax=None, col_amax=None, row_data=None, row_scale=None,
                         col_data=None, col_scale=None, stream=None):
    xp, m, k = _x(x)
    sp, e = _splits(h_splits)
    _check("nvfp4_group_quantize", load_library().nvfp4_group_quantize(
        xp, m, k, e, sp, _ptr(row_amax), _ptr(col_amax), _ptr(row_data), _ptr(row_scale),
        _ptr(col_data), _ptr(col_scale), _stream(stream)))


def nvfp4_group_amax_graphsafe(x, num_experts, d_offs, d_status, row_amax=None, col_amax=None,
                               stream=None):
    xp, m, k = _x(x)
    _check("nvfp4_group_amax_graphsafe", load_library().nvfp4_group_amax_graphsafe(
        xp, m, k, int(num_experts), _ptr(d_offs), _ptr(row_amax), _ptr(col_amax), _ptr(d_status),
        _stream(stream)))


def nvfp4_group_cast_graphsafe(x, num_experts, d_offs, d_status, row_amax=None, col_amax=None,
                               row_data=None, row_scale=None, col_data=None, col_scale=None,
                               stream=None):
    xp, m, k = _x(x)
    _check("nvfp4_group_cast_graphsafe", load_library().nvfp4_group_cast_graphsafe(
        xp, m, k, int(num_experts), _ptr(d_offs), _ptr(row_amax), _ptr(col_amax), _ptr(row_data),
        _ptr(row_scale), _ptr(col_data), _ptr(col_scale), _ptr(d_status), _stream(stream)))


def nvfp4_group_quantize_graphsafe(x, num_experts, d_offs, d_status, row_amax=None, col_amax=None,
                                   row_data=None, row_scale=None, col_data=None, col_scale=None,
                                   stream=None):
    xp, m, k = _x(x)
    _check("nvfp4_group_quantize_graphsafe", load_library().nvfp4_group_quantize_graphsafe(
        xp, m, k, int(num_experts), _ptr(d_offs), _ptr(row_amax), _ptr(col_amax), _ptr(row_data),
        _ptr(row_scale), _ptr(col_data), _ptr(col_scale), _ptr(d_status), _stream(stream)))


def nvfp4_group_dequant_rowwise(row_data, row_scale, row_amax, out, stream=None):
    """row_data [rows, k/2] u8, row_scale [rows, k/16] u8, row_amax [rows] f32 -> out [rows, k] f32."""
    rows, half_k = row_data.shape
    _check("nvfp4_group_dequant_rowwise", load_library().nvfp4_group_dequant_rowwise(
        _ptr(row_data), _ptr(row_scale), _ptr(row_amax), rows, 2 * half_k, _ptr(out), _stream(stream)))


def nvfp4_group_dequant_columnwise(col_data, col_scale, col_amax, h_splits, k, out, stream=None):
    """Transposed output (per expert [k, M_e] lines) -> out f32 in the same layout (k * sum_m values)."""
    sp, e = _splits(h_splits)
    sum_m = sum(int(v) for v in h_splits)
    _check("nvfp4_group_dequant_columnwise", load_library().nvfp4_group_dequant_columnwise(
        _ptr(col_data), _ptr(col_scale), _ptr(col_amax), sum_m, int(k), e, sp, _ptr(out), _stream(stream)))


def nvfp4_group_dequant_columnwise_graphsafe(col_data, col_scale, col_amax, m_capacity, k, num_experts, d_offs,
                                             out, d_status, stream=None):
    _check("nvfp4_group_dequant_columnwise_graphsafe",
           load_library().nvfp4_group_dequant_columnwise_graphsafe(
               _ptr(col_data), _ptr(col_scale), _ptr(col_amax), int(m_capacity), int(k), int(num_experts),
               _ptr(d_offs), _ptr(out), _ptr(d_status), _stream(stream)))


def mxfp4_group_cast(x, h_splits, row_data=None, row_scale=None, col_data=None, col_scale=None, stream=None):
    xp, m, k = _x(x)
    sp, e = _splits(h_splits)
    _check("mxfp4_group_cast", load_library().mxfp4_group_cast(
        xp, m, k, e, sp, _ptr(row_data), _ptr(row_scale), _ptr(col_data), _ptr(col_scale), _stream(stream)))


def mxfp4_group_cast_graphsafe(x, num_experts, d_offs, d_status, row_data=None, row_scale=None, col_data=None,
                               col_scale=None, stream=None):
    xp, m, k = _x(x)
    _check("mxfp4_group_cast_graphsafe", load_library().mxfp4_group_cast_graphsafe(
        xp, m, k, int(num_experts), _ptr(d_offs), _ptr(row_data), _ptr(row_scale), _ptr(col_data),
        _ptr(col_scale), _ptr(d_status), _stream(stream)))


def nvfp4_group_gemm(a_data, a_scale, a_amax, b_data, b_scale, b_amax, h_splits, out, stream=None):
    """Forward form: a_data [sum_m, k/2], a_scale [sum_m, k/16], a_amax [sum_m];
    b_data [E, n, k/2], b_scale [E, n, k/16], b_amax [E*n] -> out f32 [sum_m, n]."""
    sum_m, half_k = a_data.shape
    E, n = b_data.shape[0], b_data.shape[1]
    sp, e = _splits(h_splits)
    if e != E:
        raise ValueError(f"{e} splits for {E} expert operands")
    _check("nvfp4_group_gemm", load_library().nvfp4_group_gemm(
        _ptr(a_data), _ptr(a_scale), _ptr(a_amax), _ptr(b_data), _ptr(b_scale), _ptr(b_amax), sum_m, n,
        2 * half_k, e, sp, _ptr(out), _stream(stream)))


def nvfp4_group_gemm_graphsafe(a_data, a_scale, a_amax, b_data, b_scale, b_amax, d_offs, out, d_status,
                               stream=None):
    m_capacity, half_k = a_data.shape
    E, n = b_data.shape[0], b_data.shape[1]
    _check("nvfp4_group_gemm_graphsafe", load_library().nvfp4_group_gemm_graphsafe(
        _ptr(a_data), _ptr(a_scale), _ptr(a_amax), _ptr(b_data), _ptr(b_scale), _ptr(b_amax), m_capacity, n,
        2 * half_k, E, _ptr(d_offs), _ptr(out), _ptr(d_status), _stream(stream)))


def nvfp4_group_gemm_wgrad(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax, h_splits,
                           n, k, out, stream=None):
    """Weight-gradient form on two columnwise cast outputs (dY's with n lines
    per expert, X's with k) -> out f32 [E, n, k]."""
    sp, e = _splits(h_splits)
    sum_m = sum(int(v) for v in h_splits)
    _check("nvfp4_group_gemm_wgrad", load_library().nvfp4_group_gemm_wgrad(
        _ptr(a_col_data), _ptr(a_col_scale), _ptr(a_col_amax), _ptr(b_col_data), _ptr(b_col_scale),
        _ptr(b_col_amax), sum_m, int(n), int(k), e, sp, _ptr(out), _stream(stream)))


def nvfp4_group_gemm_wgrad_graphsafe(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax,
                                     m_capacity, num_experts, d_offs, n, k, out, d_status, stream=None):
    _check("nvfp4_group_gemm_wgrad_graphsafe", load_library().nvfp4_group_gemm_wgrad_graphsafe(
        _ptr(a_col_data), _ptr(a_col_scale), _ptr(a_col_amax), _ptr(b_col_data), _ptr(b_col_scale),
        _ptr(b_col_amax), int(m_capacity), int(n), int(k), int(num_experts), _ptr(d_offs), _ptr(out),
        _ptr(d_status), _stream(stream)))


# ---------------------------------------------------------------- helpers

def alloc_outputs(m_rows: int, k: int, num_experts: int, rowwise: bool = True, columnwise: bool = True,
                  device="cuda"):
    """Allocate the output buffers for ``m_rows`` rows (sum_m, or m_capacity)."""
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    out = {"row_amax": None, "col_amax": None, "row_data": None, "row_scale": None,
           "col_data": None, "col_scale": None}
    if rowwise:
        out.update(row_amax=torch.empty(m_rows, **f32), row_data=torch.empty((m_rows, k // 2), **u8),
                   row_scale=torch.empty((m_rows, k // 16), **u8))
    if columnwise:
        out.update(col_amax=torch.empty(num_experts * k, **f32),
                   col_data=torch.empty(m_rows * k // 2, **u8), col_scale=torch.empty(m_rows * k // 16, **u8))
    return out


def alloc_mx_outputs(m_rows: int, k: int, rowwise: bool = True, columnwise: bool = True, device="cuda"):
    """Allocate MXFP4 output buffers for ``m_rows`` rows (codes 2 per byte, one E8M0 byte per 32)."""
    u8 = dict(dtype=torch.uint8, device=device)
    out = {"row_data": None, "row_scale": None, "col_data": None, "col_scale": None}
    if rowwise:
        out.update(row_data=torch.empty((m_rows, k // 2), **u8), row_scale=torch.empty((m_rows, k // 32), **u8))
    if columnwise:
        out.update(col_data=torch.empty(m_rows * k // 2, **u8), col_scale=torch.empty(m_rows * k // 32, **u8))
    return out


def offsets_from_splits(h_splits: Sequence[int]) -> list:
    """Inclusive row ends (the graph-safe routing format)."""
    out, acc = [], 0
    for v in h_splits:
        acc += int(v)
        out.append(acc)
    return out
