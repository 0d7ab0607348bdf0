"""Shared helpers of the GPU tests: run the HIP path through the C ABI with
guard bands around every output, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from nvfp4_block_scaled_group_amd import binding as B

GUARD = 256          # bytes of canary before and after every output
CANARY = 0xA5


def log(msg: str):
    print(f"[gpu] {msg}", flush=True)


def to_device(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to("cuda:0")


class Guarded:
    """A device buffer of ``nbytes`` with canary bands on both sides."""

    def __init__(self, nbytes: int, dtype=torch.uint8, shape=None):
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda:0")
        inner = self.buf[GUARD:GUARD + nbytes]
        self.t = inner.view(dtype)
        if shape is not None:
            self.t = self.t.view(shape)

    def guards_intact(self) -> bool:
        b = self.buf.cpu().numpy()
        return bool((b[:GUARD] == CANARY).all() and (b[GUARD + self.nbytes:] == CANARY).all())

    def numpy(self) -> np.ndarray:
        return self.t.cpu().numpy()


def alloc(m_rows: int, k: int, E: int, rowwise: bool, columnwise: bool):
    out = {}
    if rowwise:
        out["row_amax"] = Guarded(4 * m_rows, torch.float32)
        out["row_data"] = Guarded(m_rows * k // 2, torch.uint8, (m_rows, k // 2))
        out["row_scale"] = Guarded(m_rows * k // 16, torch.uint8, (m_rows, k // 16))
    if columnwise:
        out["col_amax"] = Guarded(4 * E * k, torch.float32)
        out["col_data"] = Guarded(m_rows * k // 2)
        out["col_scale"] = Guarded(m_rows * k // 16)
    return out


def tensors(out):
    keys = ("row_amax", "col_amax", "row_data", "row_scale", "col_data", "col_scale")
    return {key: (out[key].t if key in out else None) for key in keys}


def run_host_split(x_dev, splits, rowwise=True, columnwise=True, entry="two_calls"):
    m, k = x_dev.shape
    out = alloc(m, k, len(splits), rowwise, columnwise)
    t = tensors(out)
    if entry == "two_calls":
        B.nvfp4_group_amax(x_dev, splits, t["row_amax"], t["col_amax"])
        B.nvfp4_group_cast(x_dev, splits, **t)
    else:
        B.nvfp4_group_quantize(x_dev, splits, **t)
    torch.cuda.synchronize()
    return out


def to_numpy(out):
    res = {key: g.numpy() for key, g in out.items()}
    for key in ("row_amax", "col_amax"):
        if key in res:
            res[key] = res[key].astype(np.float32)
    return res


def assert_guards(out):
    for key, g in out.items():
        assert g.guards_intact(), f"canary overwritten around {key}"


def first_mismatch(a: np.ndarray, b: np.ndarray):
    a = np.asarray(a).reshape(-1)
    b = np.asarray(b).reshape(-1)
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.nonzero(a != b)[0]
    if bad.size == 0:
        return None
    i = bad[0]
    return f"{bad.size} mismatches; first at flat index {i}: gpu {a[i]:#x} vs oracle {b[i]:#x}"


def assert_equal_outputs(gpu: dict, ref: dict, keys=None):
    keys = keys or [k for k in ("row_amax", "col_amax", "row_data", "row_scale", "col_data", "col_scale")
                    if k in gpu and ref.get(k) is not None]
    for key in keys:
        msg = first_mismatch(gpu[key], ref[key])
        assert msg is None, f"{key}: {msg}"
