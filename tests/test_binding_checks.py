"""The binding checks every buffer on the host (dtype, element count,
contiguity, device) and raises ValueError before anything reaches the C
library: a wrong tensor never turns into an out-of-bounds kernel access.

Runs on the CPU: the current device is taken to be the CPU and the library is
replaced by a stand-in that fails the test if any entry point is called.
"""
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B


class _NoCalls:
    def __getattr__(self, name):
        def fail(*args, **kwargs):
            raise AssertionError(f"{name} was called although an argument check should have failed")
        return fail


@pytest.fixture(autouse=True)
def cpu_device(monkeypatch):
    monkeypatch.setattr(B, "_current_device", lambda: torch.device("cpu"))
    monkeypatch.setattr(B, "load_library", lambda *a, **k: _NoCalls())
    monkeypatch.setattr(B, "_stream", lambda s: None)


M, K, E = 256, 64, 2
SPLITS = [128, 128]


def outputs(**override):
    out = B.alloc_outputs(M, K, E, True, True, device="cpu")
    out.update(override)
    return out


def x():
    return torch.zeros((M, K), dtype=torch.bfloat16)


@pytest.mark.parametrize("key,bad", [
    ("row_amax", torch.zeros(M, dtype=torch.float64)),
    ("row_amax", torch.zeros(M - 1, dtype=torch.float32)),
    ("col_amax", torch.zeros(E * K - 1, dtype=torch.float32)),
    ("row_data", torch.zeros((M, K // 2), dtype=torch.int32)),
    ("row_data", torch.zeros((M - 1, K // 2), dtype=torch.uint8)),
    ("row_scale", torch.zeros(M * K // 16 - 1, dtype=torch.uint8)),
    ("col_data", torch.zeros(M * K // 2 - 16, dtype=torch.uint8)),
    ("col_scale", torch.zeros(M * K // 8, dtype=torch.uint8)[::2]),  # not contiguous
    ("col_scale", torch.zeros(M * K // 16, dtype=torch.uint8, device="meta")),
])
@pytest.mark.parametrize("entry", ["cast", "quantize", "quantize_graphsafe", "cast_4over6", "cast_4over6_graphsafe"])
def test_bad_output_buffer_is_rejected(key, bad, entry):
    out = outputs(**{key: bad})
    offs, status = torch.tensor([128, 256], dtype=torch.int32), torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match=key):
        if entry == "cast":
            B.nvfp4_group_cast(x(), SPLITS, **out)
        elif entry == "quantize":
            B.nvfp4_group_quantize(x(), SPLITS, **out)
        elif entry == "cast_4over6":
            B.nvfp4_group_cast_4over6(x(), SPLITS, **out, scale_bound=256, err_mode=B.ERR_MSE)
        elif entry == "cast_4over6_graphsafe":
            B.nvfp4_group_cast_4over6_graphsafe(x(), E, offs, status, **out, scale_bound=256, err_mode=B.ERR_MAE)
        else:
            B.nvfp4_group_quantize_graphsafe(x(), E, torch.tensor([128, 256], dtype=torch.int32),
                                             torch.zeros(1, dtype=torch.int32), **out)


@pytest.mark.parametrize("fn", ["nvfp4_group_amax", "nvfp4_group_amax_tensor"])
def test_amax_entries_check_their_buffers(fn):
    with pytest.raises(ValueError, match="col_amax"):
        getattr(B, fn)(x(), SPLITS, torch.zeros(M), torch.zeros(E * K - 1))
    with pytest.raises(ValueError, match="row_amax"):
        getattr(B, fn)(x(), SPLITS, torch.zeros(M - 1), None)


def test_amax_buffers_checked():
    with pytest.raises(ValueError, match="col_amax"):
        B.nvfp4_group_amax(x(), SPLITS, torch.zeros(M), torch.zeros(E * K - 1))
    with pytest.raises(ValueError, match="row_amax"):
        B.nvfp4_group_amax(x(), SPLITS, torch.zeros(M, dtype=torch.float16), None)


@pytest.mark.parametrize("d_offs,d_status,key", [
    (torch.tensor([128, 256], dtype=torch.int64), torch.zeros(1, dtype=torch.int32), "d_offs"),
    (torch.tensor([128], dtype=torch.int32), torch.zeros(1, dtype=torch.int32), "d_offs"),
    (torch.tensor([128, 256], dtype=torch.int32), torch.zeros(0, dtype=torch.int32), "d_status"),
    (torch.tensor([128, 256], dtype=torch.int32), None, "d_status"),
])
def test_bad_device_routing_buffers(d_offs, d_status, key):
    with pytest.raises(ValueError, match=key):
        B.nvfp4_group_amax_graphsafe(x(), E, d_offs, d_status, torch.zeros(M), torch.zeros(E * K))
    with pytest.raises(ValueError, match=key):
        B.nvfp4_group_cast_graphsafe(x(), E, d_offs, d_status, **outputs())


def test_bad_x():
    with pytest.raises(ValueError, match="x must be"):
        B.nvfp4_group_quantize(torch.zeros(M * K, dtype=torch.bfloat16), SPLITS, **outputs())
    with pytest.raises(ValueError, match="x must be"):
        B.nvfp4_group_quantize(torch.zeros((M, K), dtype=torch.float32), SPLITS, **outputs())


def test_dequant_and_mxfp4_buffers_checked():
    rd, rs = torch.zeros((M, K // 2), dtype=torch.uint8), torch.zeros((M, K // 16), dtype=torch.uint8)
    with pytest.raises(ValueError, match="out"):
        B.nvfp4_group_dequant_rowwise(rd, rs, torch.zeros(M), torch.zeros(M * K - 1))
    with pytest.raises(ValueError, match="row_amax"):
        B.nvfp4_group_dequant_rowwise(rd, rs, torch.zeros(M - 1), torch.zeros(M * K))
    cd, cs = torch.zeros(M * K // 2, dtype=torch.uint8), torch.zeros(M * K // 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="col_amax"):
        B.nvfp4_group_dequant_columnwise(cd, cs, torch.zeros(E * K - 1), SPLITS, K, torch.zeros(M * K))
    mx = B.alloc_mx_outputs(M, K, device="cpu")
    mx["row_scale"] = torch.zeros(M * K // 32 - 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="row_scale"):
        B.mxfp4_group_cast(x(), SPLITS, **mx)


def test_gemm_operands_checked():
    n = 32
    a = (torch.zeros((M, K // 2), dtype=torch.uint8), torch.zeros(M * K // 16, dtype=torch.uint8), torch.zeros(M))
    b = (torch.zeros((E, n, K // 2), dtype=torch.uint8), torch.zeros(E * n * K // 16, dtype=torch.uint8),
         torch.zeros(E * n))
    with pytest.raises(ValueError, match="out"):
        B.nvfp4_group_gemm(*a, *b, SPLITS, torch.zeros(M * n - 1))
    with pytest.raises(ValueError, match="b_data"):
        B.nvfp4_group_gemm(*a, torch.zeros((E * n, K // 2), dtype=torch.uint8), *b[1:], SPLITS, torch.zeros(M * n))
    with pytest.raises(ValueError, match="b_amax"):
        B.nvfp4_group_gemm(*a, *b[:2], torch.zeros(E * n - 1), SPLITS, torch.zeros(M * n))
    dy = (torch.zeros(M * n // 2, dtype=torch.uint8), torch.zeros(M * n // 16, dtype=torch.uint8), torch.zeros(E * n))
    xc = (torch.zeros(M * K // 2, dtype=torch.uint8), torch.zeros(M * K // 16, dtype=torch.uint8), torch.zeros(E * K))
    with pytest.raises(ValueError, match="out"):
        B.nvfp4_group_gemm_wgrad(*dy, *xc, SPLITS, n, K, torch.zeros(E * n * K - 1))
    with pytest.raises(ValueError, match="a_col_data"):
        B.nvfp4_group_gemm_wgrad(torch.zeros(M * n // 2 - 1, dtype=torch.uint8), *dy[1:], *xc, SPLITS, n, K,
                                 torch.zeros(E * n * K))
