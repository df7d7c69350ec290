"""Host logic of bench.py, on the CPU: the algorithmic counts behind `value`
and `roofline.achieved`, the counter-to-bytes conversion behind
`roofline.traffic`, and the refusal of more than one GPU."""
import csv
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_counts_of_the_bench_workload():
    # Per token-head: bytes (2d + dv) * in + dv * out; flops 4F(dv+1) for the
    # state read-out and update with the denominator column, plus
    # (min(c, 256) + 1)(d + dv + 1) for the causal half of a c-token diagonal
    # block ("Expanding Attention", "Time" and "Memory").
    w = W.WORKLOADS["based_order2_prefill"]
    assert (w.B, w.H, w.N, w.d, w.dv, w.n_terms, w.dtype) == (4, 16, 4096, 16, 64, 3, "bf16")
    F = math.comb(w.d + w.n_terms - 1, w.n_terms - 1)
    assert F == 153
    th = 4 * 16 * 4096
    bytes_, flops, F_b = bench.algorithmic_prefill(w, chunk=32)
    assert F_b == F
    assert bytes_ == th * (2 * 16 + 64) * 2 + th * 64 * 2 == 83_886_080
    assert flops == th * (4 * 153 * 65 + 33 * 81)
    # a chunk beyond 256 tokens earns no more diagonal-block credit
    assert bench.algorithmic_prefill(w, chunk=1024)[1] == th * (4 * 153 * 65 + 257 * 81)


def test_algorithmic_counts_of_the_headline_workload():
    # the long-context order-2 workload: d = 64 gives F = 2145 features
    w = W.WORKLOADS[bench.HEADLINE]
    assert (w.B, w.H, w.N, w.d, w.dv, w.n_terms, w.dtype, w.a) == (1, 8, 65536, 64, 64, 3, "bf16", 8.0)
    bytes_, flops, F = bench.algorithmic_prefill(w, chunk=32)
    assert F == 2145 == math.comb(66, 2)
    th = 8 * 65536
    assert bytes_ == th * (2 * 64 + 64) * 2 + th * 64 * 2
    assert flops == th * (4 * 2145 * 65 + 33 * 129)


def test_oracle_sample_blocks_cover_the_sequence():
    # every block once, and the first blocks spread over the whole sequence
    order = bench._van_der_corput_blocks(256)
    assert sorted(order) == list(range(256))
    assert order[:4] == [0, 128, 64, 192]
    first = np.array(order[:16])
    assert abs(first.mean() - 127.5) < 16


def _write_pmc(dirname, counter, values):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "p_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        i = 0
        for kernel, vals in values.items():
            for v in vals:
                wr.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": v})
                i += 1


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    # The copy of 256 MiB reads FETCH_SIZE = 128 MiB and WRITE_SIZE = 256 MiB
    # (in KiB): fetch counts scale by 2, write counts by 1; the prefill's
    # counters are averaged over its dispatches.
    copy = "__amd_rocclr_copyBuffer"
    o2 = "void tl::o2::o2_kernel<true>(tl::PrefillArgs)"
    reset = "tl::o2::o2_reset(int*, int)"
    _write_pmc(tmp_path / "cf", "FETCH_SIZE", {copy: [131072.0, 131072.0], "other": [1.0]})
    _write_pmc(tmp_path / "cw", "WRITE_SIZE", {copy: [262144.0]})
    _write_pmc(tmp_path / "pf", "FETCH_SIZE", {o2: [50000.0, 52000.0], reset: [1.0]})
    _write_pmc(tmp_path / "pw", "WRITE_SIZE", {o2: [52500.0], reset: [2.0]})
    out = tmp_path / "traffic.json"
    bench.pmc_summary("based_order2_prefill", str(tmp_path / "pf"), str(tmp_path / "pw"), str(tmp_path / "cf"),
                      str(tmp_path / "cw"), str(out))
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["kernels"][o2]["fetch_bytes"] == pytest.approx(51000.0 * 1024 * 2)
    assert rec["kernels"][o2]["write_bytes"] == pytest.approx(52500.0 * 1024)
    total = (51000.0 * 2 + 52500.0 + 1.0 * 2 + 2.0) * 1024
    assert rec["bytes_per_call"] == pytest.approx(total)
    # the record is used only while the timed kernel's sources are unchanged
    monkeypatch.setattr(bench, "traffic_path", lambda name: str(out))
    assert bench.stored_traffic("based_order2_prefill") == pytest.approx(total)
    rec["source_hash"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.stored_traffic("based_order2_prefill") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
