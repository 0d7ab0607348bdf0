"""Build ``libnvfp4g.so`` (HIP for gfx950) in-tree.

    python -m nvfp4_block_scaled_group_amd.build

Compiles ``csrc/*.hip`` with hipcc for gfx950 and links a plain shared library
exporting the C ABI of ``include/nvfp4_group.h``; also builds
``probe/libhbmprobe.so`` (the benchmark's memory-ceiling kernels, not part
of that ABI).  The library's dependency on
the HIP runtime is recorded as ``libamdhip64.so`` (the name PyTorch's ROCm
build loads its own runtime under), so inside a process that already imported
torch the library binds to that same runtime instead of loading a second one;
on its own it finds ROCm's runtime through its RUNPATH.
"""
from __future__ import annotations

import glob
import importlib.util
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libnvfp4g.so")
PROBE_SRC = os.path.join(PKG, "probe", "hbm_probe.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libhbmprobe.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # each float expression is one IEEE op: no FMA contraction, no fast math
    "-ffp-contract=off", "-fno-fast-math",
    # no packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def _hip_runtime_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec and spec.submodule_search_locations:
        d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    return os.path.join(ROCM, "lib")


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    link = ["g++", "-shared", "-o", tmp, *objs, f"-L{_hip_runtime_dir()}", "-lamdhip64",
            f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    build_probe(hipcc, verbose)
    return LIB


def build_probe(hipcc: str, verbose: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, "hbm_probe.hip.o")
    cmd = [hipcc, *HIPCC_FLAGS, "-c", PROBE_SRC, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    tmp = PROBE_LIB + ".tmp"
    subprocess.check_call(["g++", "-shared", "-o", tmp, obj, f"-L{_hip_runtime_dir()}", "-lamdhip64",
                           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-Wl,--no-undefined"])
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
