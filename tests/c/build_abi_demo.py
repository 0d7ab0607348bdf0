"""Build tests/c/abi_graph_replay, the test-only C++/HIP caller of
libnvfp4g.so that uses no PyTorch (host code only; it links the built
library through a path relative to itself, so the repository can move)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from nvfp4_block_scaled_group_amd import build as B  # noqa: E402

EXE = os.path.join(HERE, "abi_graph_replay")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "abi_graph_replay.cpp")
    pkg = os.path.dirname(B.LIB)
    rel = os.path.relpath(pkg, HERE)
    tmp = EXE + ".tmp"
    cmd = ["hipcc", "-O2", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", src, "-o", tmp,
           f"-L{pkg}", "-l:" + os.path.basename(B.LIB), f"-Wl,-rpath,$ORIGIN/{rel}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
