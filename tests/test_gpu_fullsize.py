"""Parity at the full workload sizes, in the launch configuration the bench
times (bf16 output for bf16 workloads): every row where the fp64 oracle can
afford it (N <= 8192), else every row around each chunk and segment boundary
plus a seeded random set; per head and per row (tests/helpers.py)."""
import math
import sys

import numpy as np
import pytest

from oracle import taylor_oracle as T
import workloads as W
from tests.helpers import TOL, boundary_rows, check_parity, normwise_rel, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import taylor_series_linear_amd as tl  # noqa: E402



def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["order2_tiny_fp32", "based_order2_prefill", "order4_prefill",
                                  "long_order2_prefill"])
def test_prefill_workload(name):
    w = W.WORKLOADS[name]
    say("full-size prefill", name)
    x = W.make_workload(w)
    q, k, v = (to_device(x[s], w.dtype) for s in "qkv")
    out_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o, S, z = tl.prefill(q, k, v, w.n_terms, w.a, out_dtype=out_dtype, return_state=True)
    torch.cuda.synchronize()
    say("  kernel done")
    o = to_f64(o)
    assert np.all(np.isfinite(o))
    if w.N <= 8192:
        rows = np.arange(w.N)
    else:
        # both large-feature kernels use 32-token chunks and segments of a
        # multiple of 32 tokens: the chunk before and after every 1024th
        # token, two rows at every chunk edge, 1024 random rows
        rows = np.union1d(boundary_rows(w.N, 1024, span=33), boundary_rows(w.N, 32, span=1, extra=1024, seed=5))
    say(f"  oracle on {len(rows)} rows per head")
    ref = T.direct(x["q64"], x["k64"], x["v64"], w.n_terms, w.a, rows=rows)
    check_parity(o[:, :, rows], ref, w.dtype, say=say)
    # state of two heads against the oracle's
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    for b, h in heads:
        Sr, zr = T.state(x["k64"][b, h], x["v64"][b, h], w.n_terms)
        assert normwise_rel(to_f64(S[b, h])[None], Sr[None], 1) < TOL[w.dtype]
        assert normwise_rel(to_f64(z[b, h])[None, :, None], zr[None, :, None], 1) < TOL[w.dtype]


@pytest.mark.timeout(900)
def test_decode_workload():
    w = W.WORKLOADS["order2_decode"]
    say("full-size decode: generating inputs")
    x = W.make_decode_inputs(w)
    say("  uploading")
    pk = to_device(x["prefill_k"], "f32")
    pv = to_device(x["prefill_v"], "f32")
    say("  prefill of", w.N, "tokens for", w.B * w.H, "heads")
    _, S, z = tl.prefill(pk, pk, pv, w.n_terms, w.a, want_output=False, return_state=True)
    torch.cuda.synchronize()
    del pk, pv
    # steps laid out [steps, B, H, .] so each step is contiguous
    sq = to_device(np.ascontiguousarray(np.moveaxis(x["step_q"], 2, 0)), "f32")
    sk = to_device(np.ascontiguousarray(np.moveaxis(x["step_k"], 2, 0)), "f32")
    sv = to_device(np.ascontiguousarray(np.moveaxis(x["step_v"], 2, 0)), "f32")
    check_steps = [0, 1, 2, 511, w.steps - 1]
    outs = {}
    say("  decoding", w.steps, "steps")
    for s in range(w.steps):
        o = tl.decode(sq[s], sk[s], sv[s], S, z, w.n_terms, w.a)
        if s in check_steps:
            outs[s] = o.clone()
    torch.cuda.synchronize()
    say("  checking sampled heads")
    heads = [(0, 0), (17, 5), (w.B - 1, w.H - 1)]
    for (b, h) in heads:
        one = W.make_decode_inputs(w, heads=[(b, h)])
        kk = np.concatenate([one["prefill_k"][0], one["step_k"][0]]).astype(np.float64)
        vv = np.concatenate([one["prefill_v"][0], one["step_v"][0]]).astype(np.float64)
        qq = np.concatenate([np.zeros_like(one["prefill_k"][0]), one["step_q"][0]]).astype(np.float64)
        rows = [w.N + s for s in check_steps]
        ref = T.direct(qq, kk, vv, w.n_terms, w.a, rows=rows)
        got = np.stack([to_f64(outs[s][b, h]) for s in check_steps])
        check_parity(got[None], ref[None], "f32", 1, say=say, what=f"head {(b, h)}: ")
        Sr, zr = T.state(kk, vv, w.n_terms)
        assert normwise_rel(to_f64(S[b, h])[None], Sr[None], 1) < TOL["f32"]
