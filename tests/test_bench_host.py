"""Host-side logic of the benchmark and of the profile summaries it reads,
checked without a GPU: the algorithmic byte count against the sizes of the
arrays the oracle actually produces, the refusal of more than one GPU, and
the rule that a traffic figure is used only for the code it was taken on."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from nvfp4_block_scaled_group_amd import profiling, synth
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("rowwise,columnwise", [(True, True), (True, False), (False, True)])
def test_algorithmic_bytes_match_the_oracle_arrays(rowwise, columnwise):
    w = synth.random_case(5, [128, 256, 0, 128], 272, "normal")
    ref = O.group_quantize(w.x, w.splits, rowwise, columnwise)
    x_bytes = w.x.nbytes
    amax = sum(ref[n].nbytes for n in ("row_amax", "col_amax") if ref.get(n) is not None)
    outs = sum(ref[n].nbytes for n in ("row_data", "row_scale", "col_data", "col_scale")
               if ref.get(n) is not None)
    got = bench.algorithmic_bytes(w.sum_m, w.k, len(w.splits), rowwise, columnwise)
    if rowwise and not columnwise:
        # one fused pass: x read once, row amax and the rowwise output written
        assert got["step"] == x_bytes + amax + outs
    else:
        # amax pass reads x and writes the amax; the cast reads both and writes the rest
        assert got["amax_kernel"] == x_bytes + amax
        assert got["cast_kernel"] == x_bytes + amax + outs
        assert got["step"] == 2 * x_bytes + 2 * amax + outs


def test_step_bytes_of_the_expert_share_workload():
    # 32 experts, K = 7168, sum_M = 65536, both directions
    N = 65536 * 7168
    assert bench.algorithmic_bytes(65536, 7168, 32, True, True)["step"] == 2_409_889_792
    assert 2_409_889_792 == 4 * N + 2 * (4 * 65536 + 4 * 32 * 7168) + 2 * (N // 2 + N // 16)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_code_hash_ignores_comments_only():
    a = "int f() {  // first\n  return 1; /* two\n lines */\n}\n"
    b = "int f() {\n\n    return 1;\n}  // other\n"
    c = "int f() {\n  return 2;\n}\n"
    assert profiling._code(a) == profiling._code(b)
    assert profiling._code(a) != profiling._code(c)


def _summary(tmp_path, sha):
    data = {"workload": "w", "fetch_scale": 2.0, "write_scale": 1.0,
            "kernels": {"group_cast_kernel": {"fetch_bytes": 10, "write_bytes": 5, "source_sha256": sha}}}
    p = tmp_path / "s.md"
    p.write_text("# summary\n\n```json\n" + json.dumps(data) + "\n```\n")
    return str(p)


def test_traffic_is_read_only_for_the_current_code(tmp_path):
    current = profiling.source_sha256("group_cast_kernel")
    assert profiling.load_traffic(_summary(tmp_path, current), "group_cast_kernel") == \
        {"read_bytes": 10, "written_bytes": 5, "bytes": 15}
    assert profiling.load_traffic(_summary(tmp_path, "0" * 64), "group_cast_kernel") is None
    assert profiling.load_traffic(_summary(tmp_path, current), "dequant_kernel") is None
    assert profiling.load_traffic(str(tmp_path / "missing.md"), "group_cast_kernel") is None


@pytest.mark.parametrize("name", ["profiles/group_cast_kernel-deepseek_share_e32_k7168_m65536.md",
                                  "profiles/group_cast_kernel-down_proj_e64_k2048_m131072.md"])
def test_committed_summaries_parse(name):
    # each summary names the command that made it and carries per-kernel traffic
    text = open(os.path.join(ROOT, name)).read()
    assert "rocprofv3 --kernel-trace --stats" in text and "python3 bench.py" in text
    data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    cast = data["kernels"]["group_cast_kernel"]
    assert cast["fetch_bytes"] > 0 and cast["write_bytes"] > 0
    assert np.isclose(data["fetch_scale"], 2.0, rtol=0.01) and np.isclose(data["write_scale"], 1.0, rtol=0.01)
