"""CPU check of the prefill segment split and of the single-pass order-2
kernel's ticket-to-unit mapping (every wait is on a lower ticket, so every
wait ends). Compiles tests/native/sched_check.cpp against the library's
HIP-free scheduling header with the host compiler and runs it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "taylor_series_linear_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "sched_check.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_segment_split_and_ticket_mapping(tmp_path):
    exe = str(tmp_path / "sched_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
