"""Summaries of rocprofv3 runs of the benchmark, written under ``profiles/``.

    python -m nvfp4_block_scaled_group_amd.profiling \
        --stats DIR --fetch DIR --write DIR --cmd "<bench command>" --out profiles/NAME.md

``--stats`` is the output directory of ``rocprofv3 --kernel-trace --stats
--output-format csv``; ``--fetch`` and ``--write`` those of two
``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of the same command
with ``--calib-copy``, which adds a plain 1 GiB device copy.  FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) are scaled by what they read for that copy of
known size (1 GiB read, 1 GiB written), giving HBM bytes per launch.  The
summary records the SHA-256 of the HIP source it was measured on; the
benchmark reports the traffic only while the source is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(PKG, "csrc", "nvfp4_group.hip")
COPY_BYTES = 1 << 30
KERNELS = ("group_cast_kernel", "group_amax_kernel", "amax_init_kernel", "group_quantize_rowwise_kernel")


def source_sha256() -> str:
    with open(SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _short(name: str) -> str:
    for k in KERNELS:
        if k in name:
            return k
    return "copy" if "copyBuffer" in name else name.split("(")[0][-60:]


def _one(dirname: str, pattern: str) -> str:
    files = glob.glob(os.path.join(dirname, "**", pattern), recursive=True)
    if not files:
        raise FileNotFoundError(f"no {pattern} under {dirname}")
    return files[0]


def kernel_stats(dirname: str) -> dict:
    out = {}
    with open(_one(dirname, "*kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            out[_short(r["Name"])] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                                      "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    return out


def counter(dirname: str, name: str) -> dict:
    vals = {}
    with open(_one(dirname, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == name:
                vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def summarize(stats_dir: str, fetch_dir: str, write_dir: str, cmd: str, workload: str) -> tuple[str, dict]:
    st = kernel_stats(stats_dir)
    fe = counter(fetch_dir, "FETCH_SIZE")
    wr = counter(write_dir, "WRITE_SIZE")
    fscale = COPY_BYTES / (fe["copy"] * 1024.0)
    wscale = COPY_BYTES / (wr["copy"] * 1024.0)
    data = {"workload": workload, "source_sha256": source_sha256(), "fetch_scale": round(fscale, 4),
            "write_scale": round(wscale, 4), "kernels": {}}
    for k in sorted(set(fe) & set(wr)):
        if k == "copy":
            continue
        data["kernels"][k] = {"fetch_bytes": round(fe[k] * 1024 * fscale), "write_bytes": round(wr[k] * 1024 * wscale),
                              "fetch_kib_raw": fe[k], "write_kib_raw": wr[k]}
    lines = [f"# rocprofv3 summary: {workload}", "",
             "Command (run from the repository root on one MI355X):", "",
             "```", f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- {cmd}",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- {cmd}",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- {cmd}", "```", "",
             "## Kernel durations (kernel trace)", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for k, v in st.items():
        lines.append(f"| {k} | {v['calls']} | {v['avg_us']:.1f} | {v['min_us']:.1f} | {v['max_us']:.1f} |")
    lines += ["", "## HBM traffic per launch (FETCH_SIZE / WRITE_SIZE, medians over dispatches)", "",
              f"Calibration with a plain 1 GiB device copy: FETCH_SIZE reads {fe['copy']:.0f} KiB "
              f"(scale {fscale:.4f}), WRITE_SIZE reads {wr['copy']:.0f} KiB (scale {wscale:.4f}).", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes |", "|---|---|---|---|---|"]
    for k, v in data["kernels"].items():
        lines.append(f"| {k} | {v['fetch_kib_raw']:.0f} | {v['write_kib_raw']:.0f} | {v['fetch_bytes']} | "
                     f"{v['write_bytes']} |")
    lines += ["", "Machine-readable (read by bench.py; valid only for the HIP source with this SHA-256):", "",
              "```json", json.dumps(data), "```", ""]
    return "\n".join(lines), data


def load_traffic(path: str, kernel: str):
    """Bytes (read + written) per launch of `kernel` from a committed summary,
    or None if the summary is missing or was taken on a different source."""
    try:
        text = open(path).read()
    except OSError:
        return None
    block = text.split("```json", 1)[-1].split("```", 1)[0].strip() if "```json" in text else ""
    try:
        data = json.loads(block)
    except ValueError:
        return None
    if data.get("source_sha256") != source_sha256() or kernel not in data.get("kernels", {}):
        return None
    k = data["kernels"][kernel]
    return {"read_bytes": k["fetch_bytes"], "written_bytes": k["write_bytes"],
            "bytes": k["fetch_bytes"] + k["write_bytes"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--cmd", required=True)
    ap.add_argument("--workload", default="deepseek_share_e32_k7168_m65536")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    text, _ = summarize(a.stats, a.fetch, a.write, a.cmd, a.workload)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
