"""Host-side checks of the C-ABI library (no GPU): it loads, exports every
entry point declared in include/*.h, and rejects bad arguments on the host
before any HIP call is made."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "nvfp4_block_scaled_group_amd", "libnvfp4g.so")


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:nv|mx)fp4_\w+)\s*\(", text, flags=re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from nvfp4_block_scaled_group_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    assert _declared() == {
        "nvfp4_group_amax", "nvfp4_group_cast", "nvfp4_group_amax_graphsafe",
        "nvfp4_group_cast_graphsafe", "nvfp4_group_quantize", "nvfp4_group_quantize_graphsafe",
        "nvfp4_group_dequant_rowwise", "nvfp4_group_dequant_columnwise",
        "nvfp4_group_dequant_columnwise_graphsafe", "mxfp4_group_cast", "mxfp4_group_cast_graphsafe",
        "nvfp4_group_gemm", "nvfp4_group_gemm_graphsafe", "nvfp4_group_gemm_wgrad",
        "nvfp4_group_gemm_wgrad_graphsafe", "nvfp4_group_cast_4over6", "nvfp4_group_cast_4over6_graphsafe",
        "nvfp4_group_amax_tensor", "nvfp4_group_amax_tensor_graphsafe", "nvfp4_group_strerror",
    }


def test_binding_constants_match_the_header():
    """Every integer macro of the header that the binding mirrors has the
    header's value (status codes, device status bits, size limits, the
    one-launch small-input limits)."""
    from nvfp4_block_scaled_group_amd import binding
    text = open(os.path.join(ROOT, "include", "nvfp4_group.h")).read()
    checked = set()
    for name, expr in re.findall(r"#define (NVFP4G_\w+) (\(?-?[0-9]+(?: << [0-9]+)?\)?)", text):
        e = expr.strip("()")
        value = (int(e.split("<<")[0]) << int(e.split("<<")[1])) if "<<" in e else int(e)
        for attr in (name, name[len("NVFP4G_"):]):
            if hasattr(binding, attr):
                assert getattr(binding, attr) == value, (name, getattr(binding, attr), value)
                checked.add(attr)
    for name, attr in (("NVFP4G_4O6_ERR_MSE", "ERR_MSE"), ("NVFP4G_4O6_ERR_MAE", "ERR_MAE"),
                       ("NVFP4G_4O6_MAX_BOUND", "MAX_4O6_BOUND"), ("NVFP4G_4O6_DEFAULT_BOUND", "DEFAULT_4O6_BOUND")):
        value = int(re.search(r"#define %s (\d+)" % name, text).group(1))
        assert getattr(binding, attr) == value, name
        checked.add(attr)
    assert {"NVFP4G_OK", "NVFP4G_EHIP", "NVFP4G_DEV_OVERFLOW", "MAX_EXPERTS_HOST", "MAX_EXPERTS_DEVICE",
            "SMALL_MAX_EXPERT_ELEMS", "SMALL_MAX_K", "ERR_MSE", "MAX_4O6_BOUND"} <= checked


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_names_match_the_abi():
    from nvfp4_block_scaled_group_amd import binding
    for name in _declared():
        assert name in binding.EXPORTS
        if name != "nvfp4_group_strerror":
            assert callable(getattr(binding, name))


def test_strerror(lib):
    lib.nvfp4_group_strerror.restype = ctypes.c_char_p
    lib.nvfp4_group_strerror.argtypes = [ctypes.c_int]
    assert lib.nvfp4_group_strerror(0) == b"ok"
    for st in (-1, -2, -3, -4):
        assert lib.nvfp4_group_strerror(st) != b"unknown status"
    assert lib.nvfp4_group_strerror(7) == b"unknown status"


def _amax(lib, x, m, k, splits, row=None, col=None):
    f = lib.nvfp4_group_amax
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    sp = (ctypes.c_int64 * len(splits))(*splits) if splits is not None else None
    return f(x, m, k, len(splits) if splits is not None else 0, sp, row, col, None)


FAKE = 0x10000  # never dereferenced: every call below fails a host check first


@pytest.mark.parametrize("args,status", [
    ((FAKE, 256, 15, [256]), -1),            # k not a multiple of 16
    ((FAKE, 256, 0, [256]), -1),             # k = 0
    ((None, 256, 32, [256]), -1),            # NULL x with rows
    ((FAKE, -128, 32, [128]), -1),           # negative rows
    ((FAKE, 256, 32, []), -1),               # no experts
    ((FAKE, 256, 32, [100, 156]), -2),       # split not a multiple of 128
    ((FAKE, 256, 32, [128, 0]), -2),         # splits do not sum to sum_m
    ((FAKE, 256, 32, [-128, 384]), -2),      # negative split
    ((FAKE + 2, 256, 32, [256]), -3),        # misaligned x
])
def test_host_argument_checks(lib, args, status):
    x, m, k, splits = args
    assert _amax(lib, x, m, k, splits, FAKE, FAKE) == status


def test_too_many_host_experts(lib):
    assert _amax(lib, FAKE, 0, 32, [0] * 513, FAKE, FAKE) == -1


def test_cast_direction_checks(lib):
    f = lib.nvfp4_group_cast
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p] + \
        [ctypes.c_void_p] * 7
    sp = (ctypes.c_int64 * 1)(128)
    # rowwise data without its scale / amax
    assert f(FAKE, 128, 32, 1, sp, None, None, FAKE, None, None, None, None) == -1
    assert f(FAKE, 128, 32, 1, sp, None, None, FAKE, FAKE, None, None, None) == -1
    # columnwise data without col_amax
    assert f(FAKE, 128, 32, 1, sp, FAKE, None, None, None, FAKE, FAKE, None) == -1
    # misaligned output
    assert f(FAKE, 128, 32, 1, sp, FAKE, None, FAKE + 4, FAKE, None, None, None) == -3


def test_graphsafe_static_checks(lib):
    f = lib.nvfp4_group_amax_graphsafe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 5
    assert f(FAKE, 256, 32, 2, None, FAKE, FAKE, FAKE, None) == -1        # no device offsets
    assert f(FAKE, 256, 32, 2, FAKE, FAKE, FAKE, None, None) == -1        # no status word
    assert f(FAKE, 200, 32, 2, FAKE, FAKE, FAKE, FAKE, None) == -1        # capacity not %128
    assert f(FAKE, 256, 32, 0, FAKE, FAKE, FAKE, FAKE, None) == -1        # no experts
    assert f(FAKE, 256, 32, 5000, FAKE, FAKE, FAKE, FAKE, None) == -1     # too many experts


def test_dequant_host_checks(lib):
    f = lib.nvfp4_group_dequant_rowwise
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert f(FAKE, FAKE, FAKE, 128, 24, FAKE, None) == -1       # k not a multiple of 16
    assert f(None, FAKE, FAKE, 128, 32, FAKE, None) == -1       # missing input
    assert f(FAKE, FAKE, FAKE, 128, 32, FAKE + 4, None) == -3   # misaligned output
    g = lib.nvfp4_group_dequant_columnwise
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    sp = (ctypes.c_int64 * 2)(128, 100)
    assert g(FAKE, FAKE, FAKE, 228, 32, 2, sp, FAKE, None) == -2  # split not a multiple of 128


def test_mxfp4_host_checks(lib):
    f = lib.mxfp4_group_cast
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 6
    sp = (ctypes.c_int64 * 1)(128)
    assert f(FAKE, 128, 48, 1, sp, FAKE, FAKE, None, None, None) == -1         # k not a multiple of 32
    assert f(FAKE, 128, 64, 1, sp, FAKE, None, None, None, None) == -1         # rowwise data without scales
    assert f(FAKE, 128, 64, 1, sp, None, None, FAKE, None, None) == -1         # columnwise data without scales
    assert f(FAKE, 128, 64, 1, sp, FAKE, FAKE + 8, None, None, None) == -3     # misaligned scales
    bad = (ctypes.c_int64 * 1)(100)
    assert f(FAKE, 100, 64, 1, bad, FAKE, FAKE, None, None, None) == -2        # split not a multiple of 128
    g = lib.mxfp4_group_cast_graphsafe
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 7
    assert g(FAKE, 256, 64, 2, None, FAKE, FAKE, None, None, FAKE, None) == -1  # no device offsets
    assert g(FAKE, 256, 64, 2, FAKE, FAKE, FAKE, None, None, None, None) == -1  # no status word


def test_gemm_host_checks(lib):
    f = lib.nvfp4_group_gemm
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 3 + [ctypes.c_int32, ctypes.c_void_p,
                                                                   ctypes.c_void_p, ctypes.c_void_p]
    sp = (ctypes.c_int64 * 2)(128, 128)
    ok = [FAKE] * 6
    assert f(*ok, 256, 32, 96, 2, sp, FAKE, None) == -1            # k not a multiple of 128
    assert f(*ok, 256, 24, 128, 2, sp, FAKE, None) == -1           # n not a multiple of 16
    assert f(*ok, 256, 0, 128, 2, sp, FAKE, None) == -1            # n = 0
    assert f(*ok, 256, 32, 128, 2, sp, None, None) == -1           # no output
    assert f(FAKE, FAKE, None, FAKE, FAKE, FAKE, 256, 32, 128, 2, sp, FAKE, None) == -1  # no row amax
    assert f(FAKE + 8, *ok[1:], 256, 32, 128, 2, sp, FAKE, None) == -3                   # misaligned data
    assert f(*ok, 256, 32, 128, 2, sp, FAKE + 2, None) == -3       # misaligned output
    bad = (ctypes.c_int64 * 2)(128, 100)
    assert f(*ok, 228, 32, 128, 2, bad, FAKE, None) == -2          # split not a multiple of 128
    g = lib.nvfp4_group_gemm_graphsafe
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 3 + [ctypes.c_int32] + [ctypes.c_void_p] * 4
    assert g(*ok, 256, 32, 128, 2, None, FAKE, FAKE, None) == -1   # no device offsets
    assert g(*ok, 200, 32, 128, 2, FAKE, FAKE, FAKE, None) == -1   # capacity not a multiple of 128
    w = lib.nvfp4_group_gemm_wgrad
    w.restype = ctypes.c_int
    w.argtypes = f.argtypes
    assert w(*ok, 256, 24, 32, 2, sp, FAKE, None) == -1            # n not a multiple of 16
    assert w(*ok, 256, 32, 40, 2, sp, FAKE, None) == -1            # k not a multiple of 16
    assert w(*ok, 228, 32, 32, 2, bad, FAKE, None) == -2           # split not a multiple of 128
    wg = lib.nvfp4_group_gemm_wgrad_graphsafe
    wg.restype = ctypes.c_int
    wg.argtypes = g.argtypes
    assert wg(*ok, 256, 32, 32, 2, None, FAKE, FAKE, None) == -1  # no device offsets
    assert wg(*ok, 256, 32, 32, 2, FAKE, FAKE, None, None) == -1  # no status word
    assert wg(*ok, 1 << 23, 32, 32, 2, FAKE, FAKE, FAKE, None) == -1  # capacity above 2^22 rows


def test_4over6_host_checks(lib):
    """The four-over-six knobs are checked on the host: scale bound in
    1 .. 448, error mode 0 (squared) or 1 (absolute); the rest as in the cast."""
    f = lib.nvfp4_group_cast_4over6
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 5
    sp = (ctypes.c_int64 * 1)(128)
    out = [FAKE, FAKE, None, None]
    assert f(FAKE, 128, 32, 1, sp, FAKE, None, 0, 0, *out, None) == -1      # bound 0
    assert f(FAKE, 128, 32, 1, sp, FAKE, None, 449, 0, *out, None) == -1    # bound above 448
    assert f(FAKE, 128, 32, 1, sp, FAKE, None, 256, 2, *out, None) == -1    # unknown error mode
    assert f(FAKE, 128, 32, 1, sp, FAKE, None, 256, -1, *out, None) == -1
    assert f(FAKE, 128, 32, 1, sp, None, None, 256, 0, *out, None) == -1    # rowwise data without row amax
    assert f(FAKE, 128, 32, 1, sp, FAKE, None, 256, 0, FAKE + 4, FAKE, None, None, None) == -3  # misaligned
    bad = (ctypes.c_int64 * 1)(100)
    assert f(FAKE, 100, 32, 1, bad, FAKE, None, 256, 0, *out, None) == -2   # split not a multiple of 128
    g = lib.nvfp4_group_cast_4over6_graphsafe
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 6
    assert g(FAKE, 256, 32, 2, None, FAKE, None, 256, 0, *out, FAKE, None) == -1   # no device offsets
    assert g(FAKE, 256, 32, 2, FAKE, FAKE, None, 256, 0, *out, None, None) == -1   # no status word
    assert g(FAKE, 256, 32, 2, FAKE, FAKE, None, 1000, 0, *out, FAKE, None) == -1  # bound out of range


def test_amax_tensor_host_checks(lib):
    """The per-tensor amax runs the grouped amax's host checks first."""
    f = lib.nvfp4_group_amax_tensor
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 4
    sp = (ctypes.c_int64 * 2)(128, 100)
    assert f(FAKE, 228, 32, 2, sp, FAKE, FAKE, None) == -2          # split not a multiple of 128
    ok = (ctypes.c_int64 * 1)(128)
    assert f(FAKE, 128, 24, 1, ok, FAKE, FAKE, None) == -1          # k not a multiple of 16
    assert f(FAKE, 128, 32, 1, ok, FAKE + 2, None, None) == -3      # misaligned row amax
    g = lib.nvfp4_group_amax_tensor_graphsafe
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 5
    assert g(FAKE, 256, 32, 2, None, FAKE, FAKE, FAKE, None) == -1  # no device offsets
    assert g(FAKE, 256, 32, 2, FAKE, FAKE, FAKE, None, None) == -1  # no status word
