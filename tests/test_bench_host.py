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


def test_code_hash_covers_the_build_flags(monkeypatch):
    from nvfp4_block_scaled_group_amd import build
    before = profiling.source_sha256("group_cast_kernel")
    monkeypatch.setattr(build, "HIPCC_FLAGS", build.HIPCC_FLAGS + ["-DNVFP4G_STORE_AUX=2"])
    assert profiling.source_sha256("group_cast_kernel") != before


def test_code_hash_does_not_depend_on_where_the_repository_sits(monkeypatch):
    """The GPU host runs a copy of the repository at another path: the hash
    of the same code must not change with the include path's location."""
    from nvfp4_block_scaled_group_amd import build
    before = profiling.source_sha256("group_cast_kernel")
    moved = [("-I/elsewhere/include" if f.startswith("-I") else f) for f in build.HIPCC_FLAGS]
    monkeypatch.setattr(build, "HIPCC_FLAGS", moved)
    assert profiling.source_sha256("group_cast_kernel") == before


def test_every_profiled_kernel_names_an_existing_source():
    """Each kernel the summaries can list maps to a source file that exists
    (the library's kernels under csrc/, the memory-ceiling kernels under
    probe/), and kernels of one file share its hash."""
    for k, rel in profiling.KERNEL_SOURCES.items():
        assert os.path.isfile(os.path.join(profiling.PKG, rel)), (k, rel)
        assert len(profiling.source_sha256(k)) == 64
    assert profiling.source_sha256("copy_kernel") == profiling.source_sha256("read_kernel")
    assert profiling.source_sha256("copy_kernel") != profiling.source_sha256("group_cast_kernel")
    # the longer names are matched first
    assert profiling._short("(anonymous namespace)::group_cast_4o6_kernel<0>(...)") == "group_cast_4o6_kernel"
    assert profiling._short("(anonymous namespace)::cast_pattern_kernel(...)") == "cast_pattern_kernel"
    assert profiling._short("__amd_rocclr_copyBuffer") == "copy"


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


@pytest.mark.parametrize("workload", sorted(bench.TRAFFIC_FILES))
def test_committed_summaries_parse(workload):
    # each summary the bench reads names the command that made it, on the
    # same workload, and carries traffic for the kernel its file is named for
    name = bench.TRAFFIC_FILES[workload]
    text = open(os.path.join(ROOT, name)).read()
    assert "rocprofv3 --kernel-trace --stats" in text and f"python3 bench.py --workload {workload} " in text
    data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    kernel = os.path.basename(name).split("-", 1)[0]
    k = data["kernels"][kernel]
    assert k["fetch_bytes"] > 0 and k["write_bytes"] > 0
    assert np.isclose(data["fetch_scale"], 2.0, rtol=0.01) and np.isclose(data["write_scale"], 1.0, rtol=0.01)


def test_committed_summaries_match_the_current_code():
    # every kernel entry of every committed summary was taken on the code as
    # it is now (else the bench would report its traffic as unknown)
    import glob
    stale = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path).read()
        data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        for kernel, entry in data["kernels"].items():
            if entry.get("source_sha256") != profiling.source_sha256(kernel):
                stale.append((os.path.basename(path), kernel))
    assert not stale, stale


def test_four_over_six_row_accounting():
    """The four-over-six bench row: the cast kernel's byte count and the
    method's fp32 operation count (6 per element, candidate and direction)
    against the non-packed VALU issue rate (256 CUs x 4 SIMDs x 16 lanes x
    2.4 GHz), with the library replaced by a stand-in that records calls."""
    import torch

    calls = []

    class FakeB:
        DEFAULT_4O6_BOUND, ERR_MSE, ERR_MAE = 256, 0, 1

        @staticmethod
        def alloc_outputs(m, k, e, device=None):
            from nvfp4_block_scaled_group_amd import binding
            return binding.alloc_outputs(m, k, e, device="cpu")

        @staticmethod
        def nvfp4_group_cast_4over6(x, splits, **kw):
            calls.append((kw["scale_bound"], kw["err_mode"]))

    m, k, E = 256, 64, 2
    x = torch.zeros((m, k), dtype=torch.int16)
    out = FakeB.alloc_outputs(m, k, E)

    def timed(fn):
        fn()
        return 1e-5  # ms: 24 * 16384 operations at ~39 T/s

    def entry(kernel, ms, nbytes):
        return {"kernel": kernel, "ms": ms, "bytes": nbytes}

    res = bench.four_over_six_rows(FakeB, torch, timed, entry, x, [128, 128], out, E, k, m)
    assert calls == [(256, 0), (256, 1)]
    N = m * k
    for tag in ("mse", "mae"):
        r = res[f"nvfp4_group_cast_4over6_{tag}"]
        assert r["bytes"] == bench.algorithmic_bytes(m, k, E, True, True)["cast_kernel"]
        alu = r["alu"]
        assert alu["method_fp32_ops_per_launch"] == 24 * N
        assert alu["peak_Tops"] == pytest.approx(39.3216)
        assert alu["achieved_Tops"] == pytest.approx(24 * N / 1e-8 / 1e12, rel=1e-3)
        assert alu["frac"] == pytest.approx(24 * N / 1e-8 / 1e12 / 39.3216, rel=1e-3)
