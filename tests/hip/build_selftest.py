"""Build the test-only GPU self-test library tests/hip/libnvfp4g_selftest.so
(hipcc for gfx950, same flags as the product library)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from nvfp4_block_scaled_group_amd import build as B  # noqa: E402

LIB = os.path.join(HERE, "libnvfp4g_selftest.so")


def build(verbose: bool = False) -> str:
    os.makedirs(B.BUILD_DIR, exist_ok=True)
    src = os.path.join(HERE, "nvfp4_selftest.hip")
    obj = os.path.join(B.BUILD_DIR, "nvfp4_selftest.hip.o")
    cmd = ["hipcc", *B.HIPCC_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    tmp = LIB + ".tmp"
    subprocess.check_call(["g++", "-shared", "-o", tmp, obj, f"-L{B._hip_runtime_dir()}", "-lamdhip64",
                           f"-Wl,-rpath,{os.path.join(B.ROCM, 'lib')}", "-Wl,--no-undefined"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
