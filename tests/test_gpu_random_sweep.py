"""Seeded random sweep of the HIP path against the oracle, byte for byte.

Each case draws an expert count (1-40), 128-row expert sizes (empty experts
included), K (any multiple of 16 up to 4096, ragged against every tile
width), a value mix, the requested directions and the entry point (amax +
cast, the one-call quantize, their graph-safe forms with spare capacity
rows).  Sizes are capped at 2^22 elements so that the oracle finishes in a
fraction of a second.  Graph-safe cases prefill every output with a
sentinel: bytes beyond the routed rows must keep it.  Every third case also
runs the MXFP4 cast (K a multiple of 32) and every fourth the four-over-six
cast with a random bound and error mode, on the same input."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import alloc, assert_guards, first_mismatch, log, tensors, to_device, to_numpy

pytestmark = pytest.mark.gpu

N_CASES = 60
MAX_ELEMS = 1 << 22
DISTS = ("normal", "outliers", "rowscale", "student", "sparse")
ENTRIES = ("two_calls", "quantize", "graphsafe_two_calls", "graphsafe_quantize")
DIRECTIONS = ((True, True), (True, False), (False, True))
SENTINEL = 0x5A


def draw(i: int):
    rng = np.random.default_rng(7000 + i)
    E = int(rng.integers(1, 41))
    k = 16 * int(rng.integers(1, 257))
    max_units = max(1, MAX_ELEMS // (128 * k))
    # total 128-row units within the size cap, spread over the experts with
    # random weights (some experts get none)
    n_units = int(rng.integers(1, min(6 * E, max_units) + 1))
    weights = rng.dirichlet(np.full(E, 0.7))
    units = rng.multinomial(n_units, weights)
    splits = [int(u) * 128 for u in units]
    dist = DISTS[i % len(DISTS)]
    rowwise, columnwise = DIRECTIONS[i % len(DIRECTIONS)]
    entry = ENTRIES[i % len(ENTRIES)]
    spare = 128 * int(rng.integers(0, 3)) if entry.startswith("graphsafe") else 0
    return E, k, splits, dist, rowwise, columnwise, entry, spare


def run_case(x_bits, splits, k, rowwise, columnwise, entry, spare):
    E = len(splits)
    total = sum(splits)
    cap = total + spare
    xb = np.zeros((cap, k), dtype=np.uint16)
    xb[:total] = x_bits
    x = to_device(xb)
    out = alloc(cap, k, E, rowwise, columnwise)
    t = tensors(out)
    if entry.startswith("graphsafe"):
        for g in out.values():
            g.t.view(torch.uint8).fill_(SENTINEL)
        d_offs = torch.tensor(B.offsets_from_splits(splits), dtype=torch.int32, device="cuda:0")
        d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        if entry == "graphsafe_two_calls":
            B.nvfp4_group_amax_graphsafe(x, E, d_offs, d_status, t["row_amax"], t["col_amax"])
            B.nvfp4_group_cast_graphsafe(x, E, d_offs, d_status, **t)
        else:
            B.nvfp4_group_quantize_graphsafe(x, E, d_offs, d_status, **t)
        torch.cuda.synchronize()
        assert int(d_status.item()) == 0
    else:
        if entry == "two_calls":
            B.nvfp4_group_amax(x, splits, t["row_amax"], t["col_amax"])
            B.nvfp4_group_cast(x, splits, **t)
        else:
            B.nvfp4_group_quantize(x, splits, **t)
        torch.cuda.synchronize()
    assert_guards(out)
    return to_numpy(out), x


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_the_oracle(i):
    E, k, splits, dist, rowwise, columnwise, entry, spare = draw(i)
    w = synth.random_case(7000 + i, splits, k, dist)
    total = w.sum_m
    log(f"sweep {i}: E {E} K {k} rows {total} (+{spare}) {dist} rowwise {rowwise} columnwise {columnwise} {entry}")
    got, x = run_case(w.x, splits, k, rowwise, columnwise, entry, spare)
    ref = O.group_quantize(w.x, splits, rowwise, columnwise)
    sizes = {"row_amax": total, "row_data": total, "row_scale": total,            # rows
             "col_amax": E * k, "col_data": total * k // 2, "col_scale": total * k // 16}
    for key, n in sizes.items():
        if key not in got:
            continue
        g = got[key].reshape(-1) if key in ("col_amax", "col_data", "col_scale", "row_amax") else got[key]
        msg = first_mismatch(g[:n], ref[key])
        assert msg is None, f"case {i} {key}: {msg}"
        if spare:
            rest = np.ascontiguousarray(g[n:]).view(np.uint8)
            assert (rest == SENTINEL).all(), f"case {i} {key} written beyond the routed rows"

    if i % 3 == 0 and k % 32 == 0 and not spare:
        log(f"sweep {i}: MXFP4 cast")
        mx = B.alloc_mx_outputs(total, k, rowwise, columnwise, device="cuda:0")
        B.mxfp4_group_cast(x, splits, **mx)
        torch.cuda.synchronize()
        rd, rs, cd, cs = O.mxfp4_group_cast(w.x, splits, rowwise, columnwise)
        for key, want in zip(("row_data", "row_scale", "col_data", "col_scale"), (rd, rs, cd, cs)):
            if want is not None:
                msg = first_mismatch(mx[key].cpu().numpy(), want)
                assert msg is None, f"case {i} mxfp4 {key}: {msg}"

    if i % 4 == 1 and not spare:
        rng = np.random.default_rng(9000 + i)
        bound = int(rng.choice([1, 6, 100, 256, 448]))
        mode = int(rng.integers(0, 2))
        log(f"sweep {i}: four-over-six bound {bound} mode {mode}")
        o4 = B.alloc_outputs(total, k, E, rowwise, columnwise, device="cuda:0")
        B.nvfp4_group_quantize(x, splits, **o4)
        for key in ("row_data", "row_scale", "col_data", "col_scale"):
            if o4.get(key) is not None:
                o4[key].fill_(0)
        B.nvfp4_group_cast_4over6(x, splits, **o4, scale_bound=bound, err_mode=mode)
        torch.cuda.synchronize()
        ref4 = O.group_quantize_4o6(w.x, splits, bound, mode, rowwise, columnwise)
        for key in ("row_data", "row_scale", "col_data", "col_scale"):
            if ref4.get(key) is not None:
                msg = first_mismatch(o4[key].cpu().numpy(), ref4[key])
                assert msg is None, f"case {i} four-over-six {key}: {msg}"
