"""GPU parity of order 6 (n_terms = 7) at d = 16, dv = 64: feature map,
prefill (one and several segments, continuation) and decode, through the
C ABI, against the fp64 oracle.

Order 6 is the highest even truncation the positivity-floor README discusses
("The 1/2 positivity floor": minimum weight about 0.15); "Expanding
Attention: A Taylor-Series Route to Linear-Time Transformers with a Fixed
Number of Recurrent States" ("Higher orders") gives its width,
C(16 + 6, 6) = 74,613 features at d = 16. Tolerances are those of every
other instantiation (tests/helpers.py).
"""
import math
import sys

import numpy as np
import pytest

from oracle import taylor_oracle as T
import workloads as W
from tests.helpers import TOL, check_parity, normwise_rel, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("needs a GPU", allow_module_level=True)

import taylor_series_linear_amd as tl  # noqa: E402

D, DV, NT = 16, 64, 7
A = 4.0  # sqrt(d)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x, dtype):
    return to_device(x["q"], dtype), to_device(x["k"], dtype), to_device(x["v"], dtype)


def test_width():
    assert tl.feature_dim(D, NT) == 74613 == math.comb(D + NT - 1, NT - 1)
    assert tl.is_supported(D, DV, NT)
    assert not tl.is_supported(D, 16, NT)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fold", [False, True])
def test_feature_map_order6(dtype, fold):
    rows = 6
    x = W.make_qkv(1, 1, rows, D, 16, dtype, 61)
    say("order-6 feature map", dtype, fold)
    phi = tl.feature_map(to_device(x["q"][0, 0], dtype), NT, a=(A if fold else None))
    torch.cuda.synchronize()
    got = to_f64(phi)
    ref = T.phi(x["q64"][0, 0], NT, a=(A if fold else None))
    assert got.shape == ref.shape == (rows, 74613)
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert err < 2e-6, err
    # per order block: phi_m(x).phi_m(y) = (x.y)^m (multinomial theorem), and
    # with alpha folded in the whole Gram matrix is w_7(x.y/a)
    xx = x["q64"][0, 0]
    if fold:
        g = got @ got.T
        assert np.max(np.abs(g - T.taylor_weight(xx @ xx.T / A, NT))) < 1e-4 * np.max(np.abs(g))
    else:
        lo, hi = T.n_features(D, 6), T.n_features(D, 7)
        g = got[:, lo:hi] @ got[:, lo:hi].T
        want = (xx @ xx.T) ** 6
        assert np.max(np.abs(g - want)) < 1e-4 * np.max(np.abs(want))


@pytest.mark.parametrize("qk", ["l2x2", "normal"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 37, 200])
def test_prefill_order6_small(dtype, N, qk):
    B, H = 1, 2
    x = W.make_qkv(B, H, N, D, DV, dtype, 600 + N, qk)
    say("order-6 prefill", dtype, N, qk)
    o, S, z = tl.prefill(*_dev(x, dtype), NT, A, out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    ref = T.direct(x["q64"], x["k64"], x["v64"], NT, A)
    check_parity(to_f64(o), ref, dtype, say=say)
    Sr, zr = T.state(x["k64"], x["v64"], NT)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]
    assert normwise_rel(to_f64(z)[..., None], zr[..., None]) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_order6_multi_segment(dtype):
    # long enough for several segments (the split targets about 512
    # workgroups over heads x segments x 117 feature slices)
    B, H, N = 1, 1, 3000
    x = W.make_qkv(B, H, N, D, DV, dtype, 607, "l2x2")
    say("order-6 prefill multi-segment", dtype)
    o, S, z = tl.prefill(*_dev(x, dtype), NT, A, out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    ref = T.direct(x["q64"], x["k64"], x["v64"], NT, A)
    check_parity(to_f64(o), ref, dtype, say=say)
    # the final state against a direct sum over every key, one order at a time
    Sr, zr = T.state(x["k64"], x["v64"], NT)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]
    assert normwise_rel(to_f64(z)[..., None], zr[..., None]) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_order6_continuation_and_decode(dtype):
    # prefill(N1), then prefill(N2 | S, z) in place, then three decode steps:
    # every output row equals the oracle on the whole sequence
    B, H, N1, N2, ND = 1, 2, 150, 90, 3
    N = N1 + N2 + ND
    x = W.make_qkv(B, H, N, D, DV, dtype, 611, "l2x2")
    q, k, v = _dev(x, dtype)
    say("order-6 continuation + decode", dtype)
    o1, S, z = tl.prefill(q[:, :, :N1].contiguous(), k[:, :, :N1].contiguous(), v[:, :, :N1].contiguous(), NT, A,
                          out_dtype=torch.float32, return_state=True)
    o2, S, z = tl.prefill(q[:, :, N1:N1 + N2].contiguous(), k[:, :, N1:N1 + N2].contiguous(),
                          v[:, :, N1:N1 + N2].contiguous(), NT, A, S, z, out_dtype=torch.float32,
                          S=S, z=z)
    outs = [o1, o2]
    for t in range(N1 + N2, N):
        od = tl.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), S, z, NT, A,
                       out_dtype=torch.float32)
        outs.append(od[:, :, None])
    torch.cuda.synchronize()
    got = np.concatenate([to_f64(t) for t in outs], axis=2)
    ref = T.direct(x["q64"], x["k64"], x["v64"], NT, A)
    check_parity(got, ref, dtype, say=say)
    # the state after the decode steps is the state of all N tokens
    Sr, zr = T.state(x["k64"], x["v64"], NT)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]
    assert normwise_rel(to_f64(z)[..., None], zr[..., None]) < TOL[dtype]


def test_order6_decode_from_oracle_state():
    # decode from an fp64-oracle state (fp32 on the device): one step per head
    # for 3 heads, against the oracle's own decode step
    B, H, N = 1, 3, 40
    x = W.make_qkv(B, H, N + 1, D, DV, "f32", 613, "l2x2")
    S0, z0 = T.state(x["k64"][:, :, :N], x["v64"][:, :, :N], NT)
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    q, k, v = _dev(x, "f32")
    say("order-6 decode from oracle state")
    od = tl.decode(q[:, :, N].contiguous(), k[:, :, N].contiguous(), v[:, :, N].contiguous(), S, z, NT, A,
                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = T.direct(x["q64"], x["k64"], x["v64"], NT, A)[:, :, N]
    check_parity(to_f64(od)[:, :, None], ref[:, :, None], "f32", say=say)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_order6_ext_decay_and_decode(dtype):
    # the extended entry points at order 6: q/k rows normalised and scaled by
    # 2 (the order-4 workload's recipe), a decay 0.99, several segments, then
    # two decode steps with the same options; against the oracle on the
    # preprocessed rows
    B, H, N, steps, g = 1, 2, 1200, 2, 0.99
    x = W.make_qkv(B, H, N + steps, D, DV, dtype, 617, "normal")
    q, k, v = _dev(x, dtype)
    opts = dict(qk_norm=True, q_scale=2.0, k_scale=2.0, gamma=g)
    say("order-6 ext + decay + decode", dtype)
    o, S, z = tl.prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous(), NT, A,
                         out_dtype=torch.float32, return_state=True, **opts)
    outs = [tl.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), S, z, NT, A,
                      out_dtype=torch.float32, **opts) for t in range(N, N + steps)]
    torch.cuda.synchronize()
    qp = T.preprocess(x["q64"], True, 2.0)
    kp = T.preprocess(x["k64"], True, 2.0)
    ref = T.direct(qp, kp, x["v64"], NT, A, gamma=g)
    check_parity(to_f64(o), ref[:, :, :N], dtype, say=say)
    got = np.stack([to_f64(t) for t in outs], axis=2)
    check_parity(got, ref[:, :, N:], dtype, say=say, what="decode: ")
