"""CPU check of the generic prefill's choice of segments per head
(csrc/sched.hpp, choose_segments): for each case the chosen P is within
[minp, maxp], the prefix pass is chosen only for two segments with every row
in one buffer range, and no other P has a lower estimated time (rounds of
resident workgroups times chunks per segment and the earlier segments' sums
each main-launch workgroup reads, plus the segment-sum launch or the prefix
pass). Named cases: the order-4 workload (16 heads x 8 feature
slices, 256 chunks, one workgroup per compute unit) takes two segments with
a prefix pass; the d = 64 extended shape (8 heads x 9 slices, 2048 chunks)
takes 7 segments (two full rounds) rather than 4 (288 workgroups: a second
round of 32); order 6 (16 heads x 117 slices) takes one."""
import math
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "taylor_series_linear_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "segplan_check.cpp")
RHO_PRE, RHO_SUM, RHO_READ = 0.6, 0.45, 0.4


def cost(units, nch, slots, minp, P):
    rounds = lambda w: math.ceil(w / slots)
    if P == 1:
        return rounds(units) * nch
    if P == 2 and minp <= 1:
        return rounds(2 * units) * nch / (2 - RHO_PRE)
    cps = math.ceil(nch / P)
    return rounds(units * P) * (cps + (P - 1) * RHO_READ) + rounds(units * (P - 1)) * cps * RHO_SUM


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs a host C++ compiler")
    out = str(tmp_path_factory.mktemp("segplan") / "segplan_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", out], check=True)
    return out


def run(exe, cases):
    args = [str(x) for c in cases for x in c]
    lines = subprocess.run([exe] + args, capture_output=True, text=True, check=True, timeout=60).stdout.splitlines()
    return [tuple(int(x) for x in line.split("->")[1].split()) for line in lines]


def test_named_cases(exe):
    got = run(exe, [(128, 256, 256, 1, 64), (72, 2048, 256, 1, 512), (1872, 64, 256, 1, 16)])
    assert got == [(2, 1), (7, 0), (1, 0)]


def test_choice_minimises_the_estimate(exe):
    cases = []
    for units in (1, 3, 8, 16, 64, 72, 100, 128, 255, 256, 300, 512, 1000):
        for nch in (1, 4, 7, 64, 256, 1000, 2048):
            for slots in (256, 512):
                for minp in (1, 2):
                    maxp = max(nch // 4, 1)
                    cases.append((units, nch, slots, minp, maxp))
    for (units, nch, slots, minp, maxp), (P, prefix) in zip(cases, run(exe, cases)):
        hi = max(maxp, minp)
        assert minp <= P <= hi
        assert bool(prefix) == (P == 2 and minp <= 1)
        best = min(cost(units, nch, slots, minp, q) for q in range(minp, min(hi, 256) + 1))
        assert cost(units, nch, slots, minp, P) <= best * (1 + 1e-9)
