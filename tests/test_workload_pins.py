"""The seeded synthetic workloads are pinned: their routing splits and the
SHA-256 of their bf16 bytes against tests/golden/workloads.json (written by
tests/golden/make_workloads.py), and the recipes' stated properties (128-row
units, empty experts, sizes) checked directly.  Both the oracle and the GPU
path draw their inputs from these generators, so a silent change of a recipe
or of numpy's streams would change what every parity test compares."""
import hashlib
import json
import os

import numpy as np
import pytest

from nvfp4_block_scaled_group_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "workloads.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["tiny", "outliers", "deepseek_share", "down_proj", "graph_replay"])
def test_workload_bytes_and_splits_are_pinned(golden, name):
    w = synth.CONFIGS[name]()
    g = golden["workloads"][name]
    assert w.name == g["id"]
    assert list(w.x.shape) == g["shape"] and w.x.dtype == np.uint16
    assert [int(v) for v in w.splits] == g["splits"]
    assert (bool(w.rowwise), bool(w.columnwise)) == (g["rowwise"], g["columnwise"])
    assert hashlib.sha256(w.x.tobytes()).hexdigest() == g["x_sha256"]
    # every recipe: 128-row expert units that add up to the rows of x
    assert all(v % synth.ROW_ALIGN == 0 and v >= 0 for v in w.splits)
    assert int(np.sum(w.splits)) == w.x.shape[0]


def test_recipe_properties():
    # lognormal(0, 0.5) weights over 8 experts, largest remainder into 64 units
    assert synth.outliers().splits.tolist() == [896, 640, 640, 256, 2176, 1536, 768, 1280]
    # Zipf(1.1) over 32 experts with the 2 smallest empty; the largest holds 18816 rows
    s = synth.zipf_splits(np.random.default_rng(3), 32, 65536)
    assert (s == 0).sum() == 2 and s.max() == 18816 and s.sum() == 65536
    # multinomial over 1024 units of 128 rows, 64 experts
    d = np.random.default_rng(4).multinomial(1024, np.full(64, 1.0 / 64)) * 128
    assert d.min() == 1024 and d.max() == 3200


@pytest.mark.parametrize("i", [0, 1, 50, 99])
def test_replay_routings_are_pinned(golden, i):
    s = synth.replay_splits(i)
    assert [int(v) for v in s] == golden["replay_splits"][str(i)]
    assert s.sum() == 65536 and (s == 0).sum() == 2


def test_replay_routings_differ():
    # the graph is replayed under changed routing: the 100 routings are not all one
    seen = {tuple(synth.replay_splits(i).tolist()) for i in range(100)}
    assert len(seen) == 100
