"""The library keeps no state between calls: two host threads, each on its
own stream, quantizing different inputs at the same time (one through the
host-split call, the other through the graph-safe call) produce exactly the
bytes each produces alone, and those equal the oracle's."""
import threading

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_group_amd import binding as B
from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

from gpu_helpers import first_mismatch, log, to_device

pytestmark = pytest.mark.gpu

KEYS = ("row_amax", "col_amax", "row_data", "row_scale", "col_data", "col_scale")
ROUNDS = 25


def _snapshot(out):
    return {k: out[k].cpu().numpy().copy() for k in KEYS}


def _same(a, b, what):
    for k in KEYS:
        msg = first_mismatch(a[k], b[k])
        assert msg is None, f"{what} {k}: {msg}"


def test_two_threads_two_streams():
    wa = synth.random_case(61, [256, 0, 512, 128, 384], 1040, "rowscale")
    wb = synth.random_case(62, [128, 640, 0, 256], 2064, "outliers")
    xa, xb = to_device(wa.x), to_device(wb.x)
    sa, sb = [int(v) for v in wa.splits], [int(v) for v in wb.splits]
    oa = B.alloc_outputs(wa.sum_m, wa.k, len(sa), device="cuda:0")
    ob = B.alloc_outputs(wb.sum_m, wb.k, len(sb), device="cuda:0")
    d_offs = torch.tensor(B.offsets_from_splits(sb), dtype=torch.int32, device="cuda:0")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def call_a():
        B.nvfp4_group_quantize(xa, sa, **oa)

    def call_b():
        B.nvfp4_group_quantize_graphsafe(xb, len(sb), d_offs, d_status, **ob)

    # alone, on the default stream
    log("concurrency: reference runs")
    call_a()
    call_b()
    torch.cuda.synchronize()
    ref_a, ref_b = _snapshot(oa), _snapshot(ob)
    _same(ref_a, {k: np.ascontiguousarray(v) for k, v in O.group_quantize(wa.x, wa.splits).items()}, "a vs oracle")
    _same(ref_b, {k: np.ascontiguousarray(v) for k, v in O.group_quantize(wb.x, wb.splits).items()}, "b vs oracle")

    # both at once, each thread on its own stream, outputs cleared between rounds
    log("concurrency: two threads")
    start = threading.Barrier(2)
    errors = []

    def worker(call, out, stream):
        try:
            with torch.cuda.stream(stream):
                start.wait()
                for _ in range(ROUNDS):
                    for k in KEYS:
                        out[k].view(torch.uint8).fill_(0xEE)
                    call()
            stream.synchronize()
        except Exception as e:  # reported below, in the test's thread
            errors.append(repr(e))

    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    threads = [threading.Thread(target=worker, args=(call_a, oa, streams[0])),
               threading.Thread(target=worker, args=(call_b, ob, streams[1]))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    assert int(d_status.item()) == 0
    _same(_snapshot(oa), ref_a, "a concurrent vs alone")
    _same(_snapshot(ob), ref_b, "b concurrent vs alone")
