"""GPU tests of the dedicated order-2 bf16 kernels away from their usual
operating point: scales a that are not powers of two, weights and scores
beyond fp16's range, and the bounded wait between segments.

* a = 2.0 ("Expanding Attention", defaults paragraph) and a = 3.0: 1/a is not
  an fp16-exact power of two, so any step that rounds 1/a or scales in the
  wrong precision shows up; every row and the final state are checked.
* A key whose weight for the later queries of its chunk overflows fp16: the
  earlier queries of the same chunk mask it, and must come out exact (a
  masked weight is exactly 0, never inf * 0 = NaN).
* a = 1000 with |q.k| up to 7e4: the raw score overflows fp16 while
  t = q.k/a does not; t is formed in fp32, so the result must be exact.
* A forced timeout of the order-2 kernel's wait for earlier segments: every
  segment's rows are either those of a normal call or NaN, never silently
  wrong.
"""
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import taylor_oracle as T
import workloads as W
from tests.helpers import TOL, check_parity, normwise_rel, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import taylor_series_linear_amd as tl  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, flush=True)


def _bf16(x64):
    stored, exact = W.round_to(x64, "bf16")
    return stored, exact


@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("a", [2.0, 3.0])
@pytest.mark.parametrize("N", [37, 1000, 3000])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dedicated_kernels_scale_not_power_of_two(d, a, N, out):
    dv, n = 64, 3
    x = W.make_qkv(1, 2, N, d, dv, "bf16", 5000 + N + d)
    say("order-2 bf16 dedicated kernel", d, a, N, out)
    od = torch.float32 if out == "f32" else torch.bfloat16
    o, S, z = tl.prefill(to_device(x["q"], "bf16"), to_device(x["k"], "bf16"), to_device(x["v"], "bf16"), n, a,
                         out_dtype=od, return_state=True)
    torch.cuda.synchronize()
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a)
    check_parity(to_f64(o), ref, "bf16", say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n)
    assert normwise_rel(to_f64(S), Sr) < TOL["bf16"]
    assert normwise_rel(to_f64(z)[..., None], zr[..., None]) < TOL["bf16"]


@pytest.mark.parametrize("d", [16, 64])
def test_masked_weight_beyond_fp16_range(d):
    # two chunks of 32; the queries of the second chunk and key 40 are 40 e_0,
    # so q.k/a = 400 for every later query of that chunk: w = 80401 > 65504.
    # Queries 32..39 mask key 40 and must match the oracle exactly as usual.
    N, dv, n, a, p = 64, 64, 3, 4.0, 40
    rng = np.random.default_rng(6060 + d)
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, dv))
    q[0, 0, 32:] = 0.0
    q[0, 0, 32:, 0] = 40.0
    k[0, 0, p] = 0.0
    k[0, 0, p, 0] = 40.0
    (qs, q64), (ks, k64), (vs, v64) = _bf16(q), _bf16(k), _bf16(v)
    say("masked overflow, d =", d)
    o = tl.prefill(to_device(qs, "bf16"), to_device(ks, "bf16"), to_device(vs, "bf16"), n, a,
                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = to_f64(o)
    rows = np.arange(p)
    assert np.all(np.isfinite(got[0, 0, :p])), "rows before the overflowing key must stay finite"
    ref = T.direct(q64, k64, v64, n, a, rows=rows)
    check_parity(got[:, :, rows], ref, "bf16", say=say)


@pytest.mark.parametrize("d", [16, 64])
def test_large_scale_scores_beyond_fp16(d):
    # |q| = 1000, |k| = 80, every key along its own query: raw scores q.k
    # reach 8e4 (beyond fp16) on the diagonal, while t = q.k / a stays within
    # +-80 for a = 1000
    N, dv, n, a = 300, 64, 3, 1000.0
    rng = np.random.default_rng(7070 + d)
    q = rng.standard_normal((1, 2, N, d))
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    k = 80.0 * q
    q = 1000.0 * q
    v = rng.standard_normal((1, 2, N, dv))
    (qs, q64), (ks, k64), (vs, v64) = _bf16(q), _bf16(k), _bf16(v)
    say("large a, d =", d, "max |q.k|", float(np.max(np.abs(np.einsum("bhtd,bhsd->bhts", q64, k64)))))
    o, S, z = tl.prefill(to_device(qs, "bf16"), to_device(ks, "bf16"), to_device(vs, "bf16"), n, a,
                         out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    got = to_f64(o)
    assert np.max(np.abs(np.einsum("bhtd,bhtd->bht", q64, k64))) > 65504
    assert np.all(np.isfinite(got))
    check_parity(got, T.direct(q64, k64, v64, n, a), "bf16", say=say)


_CHILD = r"""
import json, sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import taylor_series_linear_amd as tl
import workloads as W
x = W.make_qkv(1, 8, 4096, 16, 64, "bf16", 8080)
to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
o, S, z = tl.prefill(to(x["q"]), to(x["k"]), to(x["v"]), 3, 4.0, out_dtype=torch.float32, return_state=True)
torch.cuda.synchronize()
np.savez(sys.argv[2], o=o.cpu().numpy(), S=S.cpu().numpy(), z=z.cpu().numpy())
print("child done", flush=True)
"""


@pytest.mark.timeout(300)
def test_segment_wait_timeout_poisons_not_corrupts(tmp_path):
    # The normal call in this process; the same call in a child process whose
    # wait bound is one poll (TAYLOR_ATTN_WAIT_SPINS=1), so later segments
    # give up on predecessors still running. Each segment's rows must equal
    # the normal call's bit for bit or be all NaN.
    x = W.make_qkv(1, 8, 4096, 16, 64, "bf16", 8080)
    q, k, v = (to_device(x[s], "bf16") for s in "qkv")
    say("wait timeout: normal call")
    o, S, z = tl.prefill(q, k, v, 3, 4.0, out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    o, S, z = to_f64(o), to_f64(S), to_f64(z)
    assert np.all(np.isfinite(o))
    out = str(tmp_path / "child.npz")
    env = dict(os.environ, TAYLOR_ATTN_WAIT_SPINS="1")
    say("wait timeout: child process with a one-poll wait bound")
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, out], env=env, capture_output=True, text=True,
                       timeout=240)
    say(r.stdout.strip()[-300:], r.stderr.strip()[-500:])
    assert r.returncode == 0
    c = np.load(out)
    co = c["o"].astype(np.float64)
    poisoned = 0
    for h in range(8):
        nan_rows = np.isnan(co[0, h]).any(axis=1)
        assert not nan_rows[0], "the first segment never waits"
        # NaN rows come in whole 32-row chunks (whole segments), all-NaN
        assert np.array_equal(nan_rows, np.isnan(co[0, h]).all(axis=1))
        starts = np.flatnonzero(np.diff(nan_rows.astype(int)) == 1) + 1
        assert np.all(starts % 32 == 0)
        ok = ~nan_rows
        assert np.array_equal(co[0, h][ok], o[0, h][ok]), "a non-poisoned row differs from the normal call"
        poisoned += int(nan_rows.sum())
        for name, ref in (("S", S), ("z", z)):
            got = c[name][0, h].astype(np.float64)
            assert np.isnan(got).all() or np.array_equal(got, ref[0, h]), name
    say(f"poisoned rows: {poisoned} of {8 * 4096}")
