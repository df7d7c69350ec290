"""GPU parity of the decayed state (S_t = gamma S_{t-1} + phi(k_t) v_t^T, the
decay of the Spanish linear-attention explainer's superposed-memory
paragraph) against the fp64 oracle, through the C ABI.

Tolerances as for the plain path: normwise relative error per head, 1e-4
for fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation.
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
CONFIGS = [(16, 16, 1), (16, 64, 1), (16, 16, 3), (16, 64, 3), (16, 16, 5), (16, 64, 5),
           (32, 16, 1), (32, 64, 1), (32, 16, 3), (32, 64, 3),
           (64, 16, 1), (64, 64, 1), (64, 16, 3), (64, 64, 3)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _qk(n):
    return "l2x2" if n == 5 else "normal"


def _prefill(x, n, a, dtype, gamma, **kw):
    q, k, v = (to_device(x[s], dtype) for s in "qkv")
    r = tl.prefill(q, k, v, n, a, gamma=gamma, **kw)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("d,dv,n", CONFIGS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,gamma", [(37, 0.5), (300, 0.95)])
def test_prefill_decayed_small(d, dv, n, dtype, N, gamma):
    a = math.sqrt(d)
    x = W.make_qkv(1, 2, N, d, dv, dtype, 300 + N, _qk(n))
    say("decayed prefill", d, dv, n, dtype, N, gamma)
    o, S, z = _prefill(x, n, a, dtype, gamma, out_dtype=torch.float32, return_state=True)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a, gamma=gamma)
    check_parity(to_f64(o), ref, dtype, say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n, gamma=gamma)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]
    assert normwise_rel(to_f64(z)[..., None], zr[..., None]) < TOL[dtype]


@pytest.mark.parametrize("d,dv,n", [(16, 64, 3), (16, 64, 5), (32, 64, 3), (64, 64, 3)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_decayed_multi_segment(d, dv, n, dtype):
    # several segments; gamma^3000 = 0.05, so earlier segments still count
    N, gamma = 3000, 0.999
    a = math.sqrt(d)
    x = W.make_qkv(1, 1, N, d, dv, dtype, 17, _qk(n))
    say("decayed prefill, multi-segment", d, dv, n, dtype)
    o, S, z = _prefill(x, n, a, dtype, gamma, out_dtype=torch.float32, return_state=True)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a, gamma=gamma)
    check_parity(to_f64(o), ref, dtype, say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n, gamma=gamma)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", [False, True])
def test_decayed_continuation(dtype, inplace):
    d, dv, n, a, gamma, N1, N2 = 16, 64, 3, 4.0, 0.998, 1500, 2100
    x = W.make_qkv(1, 2, N1 + N2, d, dv, dtype, 23)
    q, k, v = (to_device(x[s], dtype) for s in "qkv")
    part = lambda t, s, e: t[:, :, s:e].contiguous()
    say("decayed continuation", dtype, inplace)
    o1, S1, z1 = tl.prefill(part(q, 0, N1), part(k, 0, N1), part(v, 0, N1), n, a, out_dtype=torch.float32,
                            return_state=True, gamma=gamma)
    rest = (part(q, N1, N1 + N2), part(k, N1, N1 + N2), part(v, N1, N1 + N2))
    if inplace:
        o2, S2, z2 = tl.prefill(*rest, n, a, S1, z1, out_dtype=torch.float32, S=S1, z=z1, gamma=gamma)
    else:
        o2, S2, z2 = tl.prefill(*rest, n, a, S1, z1, out_dtype=torch.float32, return_state=True, gamma=gamma)
    torch.cuda.synchronize()
    full = T.direct(x["q64"], x["k64"], x["v64"], n, a, gamma=gamma)
    check_parity(to_f64(o1), full[:, :, :N1], dtype, say=say, what="first part: ")
    check_parity(to_f64(o2), full[:, :, N1:], dtype, say=say, what="continuation: ")
    Sr, zr = T.state(x["k64"], x["v64"], n, gamma=gamma)
    assert normwise_rel(to_f64(S2), Sr) < TOL[dtype]
    assert normwise_rel(to_f64(z2)[..., None], zr[..., None]) < TOL[dtype]


@pytest.mark.parametrize("d,dv,n", [(16, 64, 3), (16, 16, 5), (32, 64, 3), (64, 64, 3), (64, 16, 1)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_decayed_after_prefill(d, dv, n, dtype):
    B, H, N, steps, gamma = 2, 3, 150, 5, 0.9
    a = math.sqrt(d)
    x = W.make_qkv(B, H, N + steps, d, dv, dtype, 65, _qk(n))
    q, k, v = (to_device(x[s], dtype) for s in "qkv")
    say("decayed decode", d, dv, n, dtype)
    _, S, z = tl.prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous(), n, a,
                         want_output=False, return_state=True, gamma=gamma)
    outs = []
    for s in range(steps):
        t = N + s
        outs.append(tl.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                              S, z, n, a, out_dtype=torch.float32, gamma=gamma))
    torch.cuda.synchronize()
    got = np.stack([to_f64(o_) for o_ in outs], axis=2)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a, rows=list(range(N, N + steps)), gamma=gamma)
    check_parity(got, ref, dtype, say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n, gamma=gamma)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]


def test_decode_decayed_from_oracle_state():
    d, dv, n, a, N, gamma = 16, 64, 3, 4.0, 400, 0.97
    x = W.make_qkv(1, 4, N + 1, d, dv, "f32", 79)
    S0, z0 = T.state(x["k64"][:, :, :N], x["v64"][:, :, :N], n, gamma=gamma)
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    say("decayed decode from oracle state")
    o = tl.decode(to_device(x["q"][:, :, N], "f32"), to_device(x["k"][:, :, N], "f32"),
                  to_device(x["v"][:, :, N], "f32"), S, z, n, a, gamma=gamma)
    torch.cuda.synchronize()
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a, rows=[N], gamma=gamma)[:, :, 0]
    check_parity(to_f64(o)[:, :, None], ref[:, :, None], "f32", say=say)


@pytest.mark.parametrize("d,n", [(16, 3), (64, 3)])
def test_gamma_one_matches_plain(d, n):
    # gamma = 1 on the decayed entry point (generic kernels) against the plain
    # entry point (the dedicated kernels for these bf16 shapes)
    x = W.make_qkv(2, 2, 777, d, 64, "bf16", 12)
    say("gamma = 1 vs plain", d, n)
    o1 = _prefill(x, n, math.sqrt(d), "bf16", 1.0, out_dtype=torch.float32)
    o2 = _prefill(x, n, math.sqrt(d), "bf16", None, out_dtype=torch.float32)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, math.sqrt(d))
    check_parity(to_f64(o1), ref, "bf16", say=say)
    assert normwise_rel(to_f64(o1), to_f64(o2)) < TOL["bf16"]
