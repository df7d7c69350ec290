"""CPU check of the internal feature order of the order-4 per-token query
generator (csrc/qarrange.hpp): every canonical feature of the d = 16,
order-4 basis sits at exactly one position; in every range of 80 positions
the second 40 hold the images of the first 40 under the rotation of the
indices by 8 (mod 16), which keeps the multiplicities and so the weight;
a representative without an image is a fixed point of the rotation. The
enumeration and the rotation are computed here independently of the C++
code (itertools over non-decreasing tuples, orders ascending)."""
import itertools
import os
import shutil
import subprocess
from collections import Counter

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "taylor_series_linear_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "qarrange_check.cpp")
D, N, HALF = 16, 5, 40


@pytest.fixture(scope="module")
def arrangement(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs a host C++ compiler")
    out = str(tmp_path_factory.mktemp("qarr") / "qarrange_check")
    subprocess.run(["g++", "-std=c++20", "-O1", "-Wall", "-Werror", "-fconstexpr-ops-limit=1000000000",
                    "-I", CSRC, SRC, "-o", out], check=True)
    lines = subprocess.run([out], capture_output=True, text=True, check=True, timeout=60).stdout.splitlines()
    nA, npos = (int(x) for x in lines[0].split())
    perm = [int(line.split()[1]) for line in lines[1:1 + npos]]
    reps = [tuple(int(x) for x in line.split()[1:]) for line in lines[1 + npos:1 + npos + nA]]
    return nA, npos, perm, reps


def basis():
    return [t for m in range(N) for t in itertools.combinations_with_replacement(range(D), m)]


def rotate(t):
    return tuple(sorted((i + D // 2) % D for i in t))


def test_every_feature_once(arrangement):
    nA, npos, perm, reps = arrangement
    F = len(basis())
    assert npos % (2 * HALF) == 0 and npos >= F
    used = [c for c in perm if c >= 0]
    assert sorted(used) == list(range(F))


def test_second_half_is_the_rotation(arrangement):
    nA, npos, perm, reps = arrangement
    tuples = basis()
    index = {t: f for f, t in enumerate(tuples)}
    for r in range(npos // (2 * HALF)):
        for k in range(HALF):
            a, b = perm[2 * HALF * r + k], perm[2 * HALF * r + HALF + k]
            if a < 0:
                assert b < 0
                continue
            img = index[rotate(tuples[a])]
            if img == a:
                assert b < 0  # fixed point: no image stored
            else:
                assert b == img
                # same multiplicities, so the same sqrt-multinomial weight
                assert sorted(Counter(tuples[a]).values()) == sorted(Counter(tuples[b]).values())


def test_representatives_and_fixed_points(arrangement):
    nA, npos, perm, reps = arrangement
    tuples = basis()
    index = {t: f for f, t in enumerate(tuples)}
    fixed = [f for f, t in enumerate(tuples) if index[rotate(t)] == f]
    # orders 0, 2 and 4 have fixed points ({}, {i, i+8}, {i, i+8, j, j+8})
    assert len(fixed) == 1 + 8 + 36
    paired = [f for f, p in reps if p]
    assert paired == sorted(paired) and all(index[rotate(tuples[f])] > f for f in paired)
    assert [f for f, p in reps if not p] == fixed
    assert nA == len(paired) + len(fixed) == (len(tuples) + len(fixed)) // 2
