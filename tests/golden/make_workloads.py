"""Writes workloads.json: the routing splits and the SHA-256 of the bf16
bytes of every synthetic workload, and the routings of graph replays 0, 1,
50 and 99.  Pins the seeded generators (they hold no quantisation
arithmetic) so that a change of a recipe or of numpy's streams shows up as a
failing test instead of silently different inputs.

    python tests/golden/make_workloads.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from nvfp4_block_scaled_group_amd import synth  # noqa: E402

REPLAYS = (0, 1, 50, 99)


def main():
    out = {"workloads": {}, "replay_splits": {}}
    for name, make in synth.CONFIGS.items():
        w = make()
        out["workloads"][name] = {"id": w.name, "shape": list(w.x.shape), "splits": [int(v) for v in w.splits],
                                  "rowwise": bool(w.rowwise), "columnwise": bool(w.columnwise),
                                  "x_sha256": hashlib.sha256(w.x.tobytes()).hexdigest()}
        del w
    for i in REPLAYS:
        out["replay_splits"][str(i)] = [int(v) for v in synth.replay_splits(i)]
    # one entry per line
    lines = ["{", ' "workloads": {']
    items = list(out["workloads"].items())
    lines += [f'  "{n}": {json.dumps(v)}' + ("," if i + 1 < len(items) else "") for i, (n, v) in enumerate(items)]
    lines += [" },", ' "replay_splits": {']
    reps = list(out["replay_splits"].items())
    lines += [f'  "{n}": {json.dumps(v)}' + ("," if i + 1 < len(reps) else "") for i, (n, v) in enumerate(reps)]
    lines += [" }", "}", ""]
    with open(os.path.join(HERE, "workloads.json"), "w") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    main()
