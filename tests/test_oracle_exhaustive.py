"""Exhaustive pins of the oracle's two conversions: every non-NaN fp32 bit
pattern through oracle_e2m1_encode, and every non-negative fp32 pattern
(+0 .. +inf) through oracle_e4m3_encode, each compared with a nearest-value
search over the format's table of values written independently in
tests/c/oracle_exhaustive.c (binary search, exact distances in double, ties
to the even code, saturation at the largest finite value).  The C checker
links the built oracle library and runs on all host cores (about 5 s and
20 s on 8 cores).  A planted E2M1 or E4M3 tie-to-odd rule or a wrong
subnormal E4M3 step fails it."""
import os
import subprocess

import pytest

from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    lib = O.build() if not os.path.exists(O.LIB) else O.LIB
    exe = str(tmp_path_factory.mktemp("oracle_exhaustive") / "oracle_exhaustive")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-o", exe,
                           os.path.join(HERE, "c", "oracle_exhaustive.c"),
                           f"-L{os.path.dirname(lib)}", f"-l:{os.path.basename(lib)}",
                           f"-Wl,-rpath,{os.path.dirname(lib)}", "-lm"])
    return exe


@pytest.mark.parametrize("fmt,patterns", [("e2m1", 2**32 - (2**24 - 2)), ("e4m3", 0x7F800000 + 1)])
def test_conversion_matches_nearest_value_search_on_every_pattern(checker, fmt, patterns):
    r = subprocess.run([checker, fmt], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    last = r.stdout.strip().splitlines()[-1]
    assert last.startswith(f"{fmt}: {patterns} patterns checked, 0 mismatches"), last
