"""GPU parity of the fused query/key preprocessing (row l2-normalisation,
scales, per-head query factor; "Expanding Attention", defaults paragraph and
"Two prerequisites"), alone and with the decayed state, against the fp64
oracle applied to the preprocessed rows.

Tolerances: normwise relative error per head, 1e-4 for fp32 inputs, 2e-2 for
bf16 inputs with fp32 accumulation.
"""
import math
import sys

import numpy as np
import pytest

from oracle import taylor_oracle as T
import workloads as W
from tests.helpers import check_parity, normwise_rel, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("needs a GPU", allow_module_level=True)

import taylor_series_linear_amd as tl  # noqa: E402

TOL = {"f32": 1e-4, "bf16": 2e-2}
HEAD = [0.7, 1.3, 2.0]  # per-head query factors for H = 3

OPTIONS = {
    "norm": dict(qk_norm=True),
    "norm_x2": dict(qk_norm=True, q_scale=2.0, k_scale=2.0),   # the order-4 workload's recipe
    "norm_heads": dict(qk_norm=True, head=True),
    "scales_only": dict(q_scale=0.5, k_scale=1.5),
    "norm_decay": dict(qk_norm=True, q_scale=2.0, gamma=0.99),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _opts(spec, H):
    o = dict(spec)
    if o.pop("head", False):
        o["q_head_scale"] = torch.tensor(HEAD[:H], dtype=torch.float32, device="cuda")
    return o


def _ref_inputs(x, spec, H):
    qs = spec.get("q_scale", 1.0)
    ks = spec.get("k_scale", 1.0)
    nm = spec.get("qk_norm", False)
    hs = np.array(HEAD[:H]) if spec.get("head", False) else None
    return T.preprocess(x["q64"], nm, qs, hs), T.preprocess(x["k64"], nm, ks)


@pytest.mark.parametrize("d,dv,n", [(16, 64, 3), (16, 16, 1), (16, 64, 5), (32, 64, 3), (64, 64, 3)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("opt", sorted(OPTIONS))
def test_prefill_ext(d, dv, n, dtype, opt):
    spec = OPTIONS[opt]
    B, H, N = 1, 3, 300
    a = math.sqrt(d)
    x = W.make_qkv(B, H, N, d, dv, dtype, 500 + d, "normal")
    say("prefill ext", d, dv, n, dtype, opt)
    q, k, v = (to_device(x[s], dtype) for s in "qkv")
    o, S, z = tl.prefill(q, k, v, n, a, out_dtype=torch.float32, return_state=True, **_opts(spec, H))
    torch.cuda.synchronize()
    qp, kp = _ref_inputs(x, spec, H)
    g = spec.get("gamma", 1.0)
    ref = T.direct(qp, kp, x["v64"], n, a, gamma=g)
    check_parity(to_f64(o), ref, dtype, say=say)
    Sr, zr = T.state(kp, x["v64"], n, gamma=g)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_ext_multi_segment_and_decode(dtype):
    d, dv, n, a, N, steps = 16, 64, 3, 4.0, 3000, 4
    spec = dict(qk_norm=True, q_scale=2.0, k_scale=2.0, head=True, gamma=0.999)
    H = 2
    x = W.make_qkv(1, H, N + steps, d, dv, dtype, 61, "normal")
    q, k, v = (to_device(x[s], dtype) for s in "qkv")
    opts = _opts(spec, H)
    say("prefill ext, segments + decode", dtype)
    o, S, z = tl.prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous(), n, a,
                         out_dtype=torch.float32, return_state=True, **opts)
    outs = [tl.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), S, z, n, a,
                      out_dtype=torch.float32, **opts) for t in range(N, N + steps)]
    torch.cuda.synchronize()
    qp, kp = _ref_inputs(x, spec, H)
    rows = np.unique(np.r_[0:70, 1000:1100, 2900:3000])
    ref = T.direct(qp, kp, x["v64"], n, a, rows=rows, gamma=0.999)
    check_parity(to_f64(o)[:, :, rows], ref, dtype, say=say)
    got = np.stack([to_f64(o_) for o_ in outs], axis=2)
    ref_d = T.direct(qp, kp, x["v64"], n, a, rows=list(range(N, N + steps)), gamma=0.999)
    check_parity(got, ref_d, dtype, say=say, what="decode: ")


def test_zero_rows_stay_zero():
    # a zero query row normalises to zero: its output is the plain prefix
    # mean of v (every weight 1), like q_t = 0 in the plain method
    d, dv, n, a, N = 16, 16, 3, 4.0, 64
    x = W.make_qkv(1, 1, N, d, dv, "f32", 3, "normal")
    x["q"][0, 0, 10] = 0.0
    x["q64"][0, 0, 10] = 0.0
    q, k, v = (to_device(x[s], "f32") for s in "qkv")
    o = tl.prefill(q, k, v, n, a, qk_norm=True)
    torch.cuda.synchronize()
    want = x["v64"][0, 0, :11].mean(axis=0)
    assert np.max(np.abs(to_f64(o)[0, 0, 10] - want)) < 1e-5
