"""GPU test of taylor_attn_prefill_noalloc: called through the C ABI, its
outputs and final state equal taylor_attn_prefill's (same kernels, scratch in
the library's static array instead of a workspace) bit for bit, on two calls
in a row, the second with a smaller input, for each prefill kernel family
whose workspace fits the scratch."""
import ctypes
import sys

import numpy as np
import pytest

import workloads as W
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import taylor_series_linear_amd as tl  # noqa: E402


def say(*a):
    print(*a, flush=True)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _call(noalloc, q, k, v, B, H, N, d, dv, n, a, dt, S0=None, z0=None, inplace=False):
    L = tl.lib()
    F = tl.feature_dim(d, n)
    o = torch.full((B, H, N, dv), float("nan"), dtype=torch.float32, device="cuda")
    if inplace:
        S, z = S0, z0
    else:
        S = torch.full((B, H, F, dv), float("nan"), dtype=torch.float32, device="cuda")
        z = torch.full((B, H, F), float("nan"), dtype=torch.float32, device="cuda")
    code = tl.TAYLOR_BF16 if dt == "bf16" else tl.TAYLOR_F32
    stream = tl._stream()
    if noalloc:
        st = L.taylor_attn_prefill_noalloc(_p(q), _p(k), _p(v), code, B, H, N, d, dv, n, a, _p(S0), _p(z0), _p(o),
                                           tl.TAYLOR_F32, _p(S), _p(z), stream)
    else:
        wsb = L.taylor_attn_prefill_workspace(B, H, N, d, dv, n, code)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        st = L.taylor_attn_prefill(_p(q), _p(k), _p(v), code, B, H, N, d, dv, n, a, _p(S0), _p(z0), _p(o),
                                   tl.TAYLOR_F32, _p(S), _p(z), _p(ws), wsb, stream)
    tl.check(st)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu(), z.cpu()


# (B, H, N, d, dv, n, dtype): the order-2 d = 16 kernel (single pass with
# tickets, several segments), the order-2 d = 64 kernel, the generic kernel
CASES = [((2, 8, 4096, 16, 64, 3, "bf16"), (1, 3, 1000, 16, 64, 3, "bf16")),
         ((1, 4, 8192, 64, 64, 3, "bf16"), (1, 2, 700, 64, 64, 3, "bf16")),
         ((1, 2, 3000, 16, 64, 5, "bf16"), (1, 1, 333, 16, 64, 5, "bf16")),
         ((2, 3, 2000, 16, 16, 3, "f32"), (1, 2, 100, 16, 16, 3, "f32"))]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_equals_workspace_call(first, second):
    for i, (B, H, N, d, dv, n, dt) in enumerate((first, second)):
        say("no-alloc prefill, call", i + 1, (B, H, N, d, dv, n, dt))
        x = W.make_qkv(B, H, N, d, dv, dt, 9100 + 7 * i + N)
        q, k, v = (to_device(x[s], dt) for s in "qkv")
        a = float(np.sqrt(d))
        ref = _call(False, q, k, v, B, H, N, d, dv, n, a, dt)
        got = _call(True, q, k, v, B, H, N, d, dv, n, a, dt)
        for name, r, g in zip("oSz", ref, got):
            assert torch.isfinite(r).all(), name
            assert torch.equal(r, g), f"{name} differs from the workspace call"


def test_noalloc_continuation_in_place():
    # S0/z0 aliasing S/z: the final state goes through the scratch too
    B, H, N1, N2, d, dv, n = 1, 8, 2000, 3000, 16, 64, 3
    x = W.make_qkv(B, H, N1 + N2, d, dv, "bf16", 9200)
    q, k, v = (to_device(x[s], "bf16") for s in "qkv")
    part = lambda t, s, e: t[:, :, s:e].contiguous()
    say("no-alloc prefill, in-place continuation")
    _, S1, z1 = _call(True, part(q, 0, N1), part(k, 0, N1), part(v, 0, N1), B, H, N1, d, dv, n, 4.0, "bf16")
    rest = [part(t, N1, N1 + N2) for t in (q, k, v)]
    Sa, za = S1.cuda(), z1.cuda()
    Sb, zb = S1.cuda(), z1.cuda()
    ref_o, _, _ = _call(False, *rest, B, H, N2, d, dv, n, 4.0, "bf16", Sa, za, inplace=True)
    got_o, _, _ = _call(True, *rest, B, H, N2, d, dv, n, 4.0, "bf16", Sb, zb, inplace=True)
    assert torch.isfinite(ref_o).all()
    assert torch.equal(got_o, ref_o)
    assert torch.equal(Sa, Sb) and torch.equal(za, zb)
