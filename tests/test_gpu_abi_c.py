"""The C ABI from a C++/HIP caller that uses no PyTorch (tests/c/abi_graph_replay,
built by build()): hipMalloc'd buffers, one hipGraph capture of
nvfp4_group_quantize_graphsafe, replayed under several routings (issue 3649
page, Description: the graph-safe calls read the routing from device
offsets, so one capture replays under changed routing).  Every replay's
amax, FP4 bytes and E4M3 scales must equal the oracle's for that routing,
rows and columnwise bytes beyond the routed total must keep the sentinel
byte, the device status must be 0, the library must refuse K = 15 on the
host before launching anything, and the capture must hold kernel nodes only."""
import os
import subprocess

import numpy as np
import pytest

from nvfp4_block_scaled_group_amd import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c", "abi_graph_replay")
SENTINEL = 0xA5

# (capacity rows, K, routings): each routing is E 128-aligned splits whose
# total may stay below the capacity; zero-row experts included.  The second
# case is small enough for the single-launch path.
CASES = [
    (1024, 272, [[256, 384, 0, 384], [128, 0, 512, 128], [0, 0, 0, 128], [1024, 0, 0, 0]]),
    (256, 128, [[128, 0, 128], [0, 128, 0], [0, 0, 0]]),
]


def _run(tmp_path, m_cap, k, routings, seed):
    E = len(routings[0])
    x = synth.random_case(seed, [m_cap], k, "rowscale").x
    offs = np.cumsum(np.asarray(routings, dtype=np.int64), axis=1).astype(np.int32)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([m_cap, k, E, len(routings)], dtype=np.int64).tobytes())
        f.write(offs.tobytes())
        f.write(np.ascontiguousarray(x).tobytes())
    print(f"[gpu] C ABI graph replay: m_cap {m_cap} k {k} E {E} routings {len(routings)}", flush=True)
    r = subprocess.run([EXE, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "refused K = 15" in r.stdout
    # the capture holds kernels only (the program fails otherwise)
    assert any(line.startswith("captured ") and line.endswith(" kernels") for line in r.stdout.splitlines())
    return x, r.stdout, np.fromfile(outp, dtype=np.uint8)


@pytest.mark.parametrize("m_cap,k,routings", CASES)
def test_c_caller_graph_replays_match_the_oracle(tmp_path, m_cap, k, routings):
    if not os.path.exists(EXE):
        pytest.fail("tests/c/abi_graph_replay is not built: run __graft_entry__.build()")
    E = len(routings[0])
    x, log, raw = _run(tmp_path, m_cap, k, routings, seed=31 + k)
    sizes = [("status", 4), ("row_amax", 4 * m_cap), ("col_amax", 4 * E * k), ("row_data", m_cap * k // 2),
             ("row_scale", m_cap * k // 16), ("col_data", m_cap * k // 2), ("col_scale", m_cap * k // 16)]
    per = sum(n for _, n in sizes)
    assert raw.size == per * len(routings)
    for i, splits in enumerate(routings):
        rec, pos = {}, i * per
        for name, n in sizes:
            rec[name] = raw[pos:pos + n]
            pos += n
        assert rec["status"].view(np.int32)[0] == 0, (i, log)
        total = int(sum(splits))
        ref = O.group_quantize(x[:total], splits)
        # routed part: the oracle's bytes; the rest: untouched
        routed = {"row_amax": 4 * total, "col_amax": 4 * E * k, "row_data": total * k // 2,
                  "row_scale": total * k // 16, "col_data": total * k // 2, "col_scale": total * k // 16}
        for name, n in routed.items():
            got = rec[name]
            want = np.ascontiguousarray(ref[name]).view(np.uint8).reshape(-1)
            assert want.size == n, (name, want.size, n)
            assert np.array_equal(got[:n], want), f"replay {i} {name} differs from the oracle"
            assert (got[n:] == SENTINEL).all(), f"replay {i} {name} written beyond the routed rows"
