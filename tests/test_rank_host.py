"""CPU check of the library's runtime feature decoder (csrc/rank.hpp), which
the order-6 kernels use in place of a compile-time basis table: for several
(d, n_terms) every index must decode to the canonical monomial (orders
ascending, non-decreasing tuples in lexicographic order, as enumerated by
itertools) with weight sqrt(m! / prod c_i!)."""
import itertools
import math
import os
import shutil
import subprocess
from collections import Counter

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "taylor_series_linear_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "rank_check.cpp")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs a host C++ compiler")
    out = str(tmp_path_factory.mktemp("rank") / "rank_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", out], check=True)
    return out


def enumerate_basis(d, n):
    for m in range(n):
        for tup in itertools.combinations_with_replacement(range(d), m):
            mult = math.factorial(m)
            for c in Counter(tup).values():
                mult //= math.factorial(c)
            yield m, math.sqrt(mult), tup


@pytest.mark.parametrize("mode", ["decode", "step"])
@pytest.mark.parametrize("d,n", [(1, 7), (2, 7), (3, 5), (4, 7), (5, 3), (16, 5), (16, 7), (64, 3)])
def test_decoder_matches_enumeration(exe, d, n, mode):
    want = list(enumerate_basis(d, n))
    args = [exe, str(d), str(n), str(len(want))] + (["step"] if mode == "step" else [])
    r = subprocess.run(args, capture_output=True, text=True, timeout=120, check=True)
    lines = r.stdout.splitlines()
    assert len(lines) == len(want)
    for line, (m, w, tup) in zip(lines, want):
        parts = line.split()
        assert int(parts[1]) == m, line
        assert tuple(int(x) for x in parts[3:]) == tup, line
        assert abs(float(parts[2]) - w) <= 1e-6 * w, line
