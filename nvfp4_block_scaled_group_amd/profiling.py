"""Summaries of rocprofv3 runs of the benchmark, written under ``profiles/``.

    python -m nvfp4_block_scaled_group_amd.profiling \
        --stats DIR --fetch DIR --write DIR --cmd "<bench command>" --out profiles/NAME.md

``--stats`` is the output directory of ``rocprofv3 --kernel-trace --stats
--output-format csv``; ``--fetch`` and ``--write`` those of two
``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of the same command
with ``--calib-copy``, which adds a plain 1 GiB device copy; each optional
``--counters DIR`` is a further ``--pmc`` run whose counters are tabulated per
kernel (medians over dispatches), with the ratios they give where the
counters are present.  GRBM_GUI_ACTIVE reads the sum over the 8 XCDs, so the
kernel's busy cycles are GRBM_GUI_ACTIVE / 8: memory-unit busy =
TA_BUSY_avr / (GRBM_GUI_ACTIVE / 8) (TA_BUSY_avr is the per-CU average),
waves waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES, VALU busy =
SQ_ACTIVE_INST_VALU * 4 / (1024 SIMDs * GRBM_GUI_ACTIVE / 8).  FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) are scaled by what they read for that copy of
known size (1 GiB read, 1 GiB written), giving HBM bytes per launch.  Each
kernel's entry records the SHA-256 of the sources it is built from (its .hip
file and the shared headers, comments aside, and the build flags); the benchmark reports a
kernel's traffic only while that code is unchanged.  ``--kernels`` limits a summary to some
kernels (plus the calibration copy).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ABI_HEADER = os.path.join(os.path.dirname(PKG), "include", "nvfp4_group.h")
COPY_BYTES = 1 << 30
# kernel -> the .hip file that defines it (relative to the package); the
# longer names come first, since names are matched as substrings of the
# profiler's kernel names.  The probe kernels are the memory-ceiling kernels
# the benchmark times beside the library's.
KERNEL_SOURCES = {
    "mxfp4_group_cast_kernel": "csrc/mxfp4_group.hip",
    "group_cast_4o6_kernel": "csrc/nvfp4_4over6.hip",
    "amax_tensor_kernel": "csrc/nvfp4_amax_tensor.hip",
    "group_cast_kernel": "csrc/nvfp4_group.hip",
    "group_amax_kernel": "csrc/nvfp4_group.hip",
    "group_amax_rows_kernel": "csrc/nvfp4_group.hip",
    "amax_init_kernel": "csrc/nvfp4_group.hip",
    "group_quantize_rowwise_kernel": "csrc/nvfp4_group.hip",
    "group_quantize_small_kernel": "csrc/nvfp4_group.hip",
    "dequant_kernel": "csrc/nvfp4_dequant.hip",
    "gemm_fwd_kernel": "csrc/nvfp4_gemm.hip",
    "gemm_wgrad_kernel": "csrc/nvfp4_gemm.hip",
    "cast_pattern_kernel": "probe/hbm_probe.hip",
    "read_kernel": "probe/hbm_probe.hip",
    "fill_kernel": "probe/hbm_probe.hip",
    "copy_kernel": "probe/hbm_probe.hip",
    "mix_kernel": "probe/hbm_probe.hip",
}
KERNELS = tuple(KERNEL_SOURCES)


def _code(text: str) -> str:
    """Source text without comments, blank lines and indentation: what the
    compiler sees, so that editing a comment keeps a measurement valid."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.strip() for line in text.splitlines() if line.strip())


def source_sha256(kernel: str) -> str:
    """SHA-256 over the code of the kernel's .hip file, the shared headers,
    the C ABI header (its macros set sizes the kernels use) and the compiler
    flags the library is built with (a -D or -O change changes the code; the
    include paths, which depend on where the repository sits, are left out)."""
    from . import build
    h = hashlib.sha256()
    # include paths name where the repository sits, not what is compiled
    flags = [f for f in build.HIPCC_FLAGS if not f.startswith("-I")]
    h.update(("flags\0" + " ".join(flags) + "\0").encode())
    paths = ([os.path.join(PKG, KERNEL_SOURCES[kernel])] +
             [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hpp")] + [ABI_HEADER])
    for path in paths:
        with open(path) as f:
            h.update(os.path.basename(path).encode() + b"\0" + _code(f.read()).encode())
    return h.hexdigest()


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
    """Median of a counter over each kernel's dispatches; for the copy kernel
    the largest dispatch, which is the 1 GiB calibration copy (the benchmark
    makes other, small device copies)."""
    vals = {}
    with open(_one(dirname, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == name:
                vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: (max(v) if k == "copy" else statistics.median(v)) for k, v in vals.items()}


SIMDS = 256 * 4  # MI355X: 256 compute units x 4 SIMDs
XCDS = 8


def all_counters(dirname: str) -> dict:
    """kernel -> counter -> median over that kernel's dispatches."""
    vals = {}
    with open(_one(dirname, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            vals.setdefault(_short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    return {k: {c: statistics.median(v) for c, v in cs.items()} for k, cs in vals.items()}


def counter_ratios(c: dict) -> dict:
    out = {}
    gui = c.get("GRBM_GUI_ACTIVE", 0) / XCDS
    if "TA_BUSY_avr" in c and gui:
        out["mem_unit_busy"] = c["TA_BUSY_avr"] / gui
    if "SQ_WAIT_ANY" in c and c.get("SQ_WAVE_CYCLES"):
        out["waves_waiting"] = c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]
    if "SQ_WAIT_INST_ANY" in c and c.get("SQ_WAVE_CYCLES"):
        out["waves_waiting_on_issue"] = c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]
    if "SQ_ACTIVE_INST_VALU" in c and gui:
        out["valu_busy"] = c["SQ_ACTIVE_INST_VALU"] * 4 / (SIMDS * gui)
    return out


def summarize(stats_dir: str, fetch_dir: str, write_dir: str, cmd: str, workload: str,
              kernels=None, counter_dirs=()) -> tuple[str, dict]:
    keep = (lambda k: True) if not kernels else (lambda k: k in kernels or k == "copy")
    st = {k: v for k, v in kernel_stats(stats_dir).items() if keep(k)}
    fe = {k: v for k, v in counter(fetch_dir, "FETCH_SIZE").items() if keep(k)}
    wr = {k: v for k, v in counter(write_dir, "WRITE_SIZE").items() if keep(k)}
    fscale = COPY_BYTES / (fe["copy"] * 1024.0)
    wscale = COPY_BYTES / (wr["copy"] * 1024.0)
    data = {"workload": workload, "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4), "kernels": {}}
    for k in sorted(set(fe) & set(wr)):
        if k not in KERNEL_SOURCES:
            continue
        data["kernels"][k] = {"fetch_bytes": round(fe[k] * 1024 * fscale), "write_bytes": round(wr[k] * 1024 * wscale),
                              "fetch_kib_raw": fe[k], "write_kib_raw": wr[k], "source_sha256": source_sha256(k)}
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
    extra = {}
    for d in counter_dirs:
        for k, cs in all_counters(d).items():
            if keep(k) and k in KERNEL_SOURCES:
                extra.setdefault(k, {}).update(cs)
    if extra:
        names = sorted({c for cs in extra.values() for c in cs})
        lines += ["", "## Other counters (medians over dispatches) and the ratios they give", "",
                  "```"] + [f"rocprofv3 --pmc {' '.join(sorted(all_counters(d)[next(iter(all_counters(d)))]))} "
                            f"--output-format csv -d <dir> -o run -- {cmd}" for d in counter_dirs] + ["```", "",
                  "| kernel | " + " | ".join(names) + " | mem unit busy | waves waiting | VALU busy |",
                  "|---" * (len(names) + 4) + "|"]
        for k, cs in extra.items():
            r = counter_ratios(cs)
            fmt = lambda v: f"{v:.3f}" if v is not None else "-"
            lines.append(f"| {k} | " + " | ".join(f"{cs[n]:.4g}" if n in cs else "-" for n in names) +
                         f" | {fmt(r.get('mem_unit_busy'))} | {fmt(r.get('waves_waiting'))} | "
                         f"{fmt(r.get('valu_busy'))} |")
            data["kernels"].setdefault(k, {})["counters"] = cs
            data["kernels"][k]["ratios"] = {n: round(v, 4) for n, v in r.items()}
    lines += ["", "Machine-readable (read by bench.py; a kernel's entry is valid only while its sources "
              "have the SHA-256 it records):", "",
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
    k = data.get("kernels", {}).get(kernel)
    if k is None or kernel not in KERNEL_SOURCES or k.get("source_sha256") != source_sha256(kernel):
        return None
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
    ap.add_argument("--kernels", default="", help="comma-separated kernel names to keep (default: all)")
    ap.add_argument("--counters", action="append", default=[], help="output dir of a further --pmc run")
    a = ap.parse_args()
    kernels = [k for k in a.kernels.split(",") if k] or None
    text, _ = summarize(a.stats, a.fetch, a.write, a.cmd, a.workload, kernels, a.counters)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
