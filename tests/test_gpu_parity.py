"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: normwise relative error per head (max over heads) 1e-4 for fp32
inputs and 2e-2 for bf16 inputs with fp32 accumulation, and a per-row bound
on every checked row (tests/helpers.py).
"""
import ctypes
import math
import sys

import numpy as np
import pytest

from oracle import taylor_oracle as T
import workloads as W
from tests.helpers import TOL, check_parity, normwise_rel, rowwise_rel, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("needs a GPU", allow_module_level=True)

import taylor_series_linear_amd as tl  # noqa: E402

CONFIGS = [(16, 16, 1), (16, 64, 1), (16, 16, 3), (16, 64, 3), (16, 16, 5), (16, 64, 5),
           (32, 16, 1), (32, 64, 1), (32, 16, 3), (32, 64, 3),
           (64, 16, 1), (64, 64, 1), (64, 16, 3), (64, 64, 3)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(B, H, N, d, dv, dtype, seed, qk="normal"):
    return W.make_qkv(B, H, N, d, dv, dtype, seed, qk)


def _run_prefill(x, n, a, dtype, **kw):
    q = to_device(x["q"], dtype)
    k = to_device(x["k"], dtype)
    v = to_device(x["v"], dtype)
    r = tl.prefill(q, k, v, n, a, **kw)
    torch.cuda.synchronize()
    return r


def _qk_kind(d, n):
    # order-4 keeps |q.k/a| <= 1 as the workloads do (rows at norm 2, a = 4)
    return "l2x2" if n == 5 else "normal"


@pytest.mark.parametrize("d,n", [(16, 1), (16, 3), (16, 5), (32, 1), (32, 3), (64, 1), (64, 3)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fold", [False, True])
def test_feature_map(d, n, dtype, fold):
    rows = 37
    x = W.make_qkv(1, 1, rows, d, 16, dtype, 11)
    say("feature_map", d, n, dtype, fold)
    phi = tl.feature_map(to_device(x["q"][0, 0], dtype), n, a=(math.sqrt(d) if fold else None))
    torch.cuda.synchronize()
    ref = T.phi(x["q64"][0, 0], n, a=(math.sqrt(d) if fold else None))
    err = np.max(np.abs(to_f64(phi) - ref)) / np.max(np.abs(ref))
    assert err < 2e-6, err
    # Gram identity on the device output: phi(x).phi(y) = w_n(x.y/a) (folded)
    if fold:
        g = to_f64(phi) @ to_f64(phi).T
        t = x["q64"][0, 0] @ x["q64"][0, 0].T / math.sqrt(d)
        assert np.max(np.abs(g - T.taylor_weight(t, n))) < 1e-4 * np.max(np.abs(g))


@pytest.mark.parametrize("d,n", [(16, 3), (16, 5), (64, 3)])
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_feature_map_unaligned_output(d, n, offset):
    # the output pointer 4, 8 or 12 bytes past a 16-byte boundary: the kernel
    # aligns its 16-byte stores to the pointer, and the floats around the
    # output stay untouched; 70 rows (more than one 64-row block, ragged)
    rows = 70
    x = W.make_qkv(1, 1, rows, d, 16, "bf16", 13)
    F = tl.feature_dim(d, n)
    buf = torch.full((rows * F + 8,), 7.0, dtype=torch.float32, device="cuda")
    xd = to_device(x["q"][0, 0], "bf16")
    say("feature_map unaligned", d, n, offset)
    tl.check(tl.lib().taylor_feature_map(ctypes.c_void_p(xd.data_ptr()), tl.TAYLOR_BF16, rows, d, n, 0.0, 0,
                                         ctypes.c_void_p(buf.data_ptr() + 4 * offset), tl._stream()))
    torch.cuda.synchronize()
    out = buf.double().cpu().numpy()
    ref = T.phi(x["q64"][0, 0], n).reshape(-1)
    got = out[offset:offset + rows * F]
    assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) < 2e-6
    assert np.all(out[:offset] == 7.0) and np.all(out[offset + rows * F:] == 7.0)


@pytest.mark.parametrize("d,dv,n", CONFIGS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 37, 64, 200, 1000])
def test_prefill_small(d, dv, n, dtype, N):
    B, H = 1, 2
    a = math.sqrt(d)
    x = _inputs(B, H, N, d, dv, dtype, 100 + N, _qk_kind(d, n))
    say("prefill", d, dv, n, dtype, N)
    o, S, z = _run_prefill(x, n, a, dtype, out_dtype=torch.float32, return_state=True)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a)
    check_parity(to_f64(o), ref, dtype, say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]
    assert normwise_rel(to_f64(z)[..., None], zr[..., None]) < TOL[dtype]


@pytest.mark.parametrize("d,dv,n", [(16, 64, 3), (16, 16, 1), (32, 64, 3), (64, 64, 3), (16, 64, 5)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_multi_segment(d, dv, n, dtype):
    # long enough that the sequence is split into several segments
    B, H, N = 1, 1, 3000
    a = math.sqrt(d)
    x = _inputs(B, H, N, d, dv, dtype, 7, _qk_kind(d, n))
    say("prefill multi-segment", d, dv, n, dtype)
    o, S, z = _run_prefill(x, n, a, dtype, out_dtype=torch.float32, return_state=True)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a)
    check_parity(to_f64(o), ref, dtype, say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]


@pytest.mark.parametrize("B,H", [(1, 8), (2, 8), (3, 5)])
def test_order2_prefill_head_groups(B, H):
    # The order-2 d=16 bf16 kernel splits each head into segments and, when
    # B*H is a multiple of 8, hands out work per group of workgroups (one
    # ticket counter per blockIdx % 8); 3 x 5 heads take the single-counter
    # path. Every row and the final state are checked against the oracle, on
    # a ragged length that leaves a partial last chunk.
    N, d, dv, n = 1100, 16, 64, 3
    a = math.sqrt(d)
    x = _inputs(B, H, N, d, dv, "bf16", 4100 + 10 * B + H)
    say("order-2 head groups", B, H)
    o, S, z = _run_prefill(x, n, a, "bf16", out_dtype=torch.float32, return_state=True)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a)
    check_parity(to_f64(o), ref, "bf16", say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n)
    assert normwise_rel(to_f64(S), Sr) < TOL["bf16"]
    assert normwise_rel(to_f64(z)[..., None], zr[..., None]) < TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("N1,N2", [(100, 37), (1500, 2100)])
def test_continuation(dtype, inplace, N1, N2):
    d, dv, n, a = 16, 64, 3, 4.0
    x = _inputs(1, 2, N1 + N2, d, dv, dtype, 21)
    q, k, v = (to_device(x[s], dtype) for s in "qkv")
    say("continuation", dtype, inplace, N1, N2)
    o1, S1, z1 = tl.prefill(q[:, :, :N1].contiguous(), k[:, :, :N1].contiguous(), v[:, :, :N1].contiguous(),
                            n, a, out_dtype=torch.float32, return_state=True)
    if inplace:
        o2, S2, z2 = tl.prefill(q[:, :, N1:].contiguous(), k[:, :, N1:].contiguous(), v[:, :, N1:].contiguous(),
                                n, a, S1, z1, out_dtype=torch.float32, S=S1, z=z1)
        assert S2.data_ptr() == S1.data_ptr()
    else:
        o2, S2, z2 = tl.prefill(q[:, :, N1:].contiguous(), k[:, :, N1:].contiguous(), v[:, :, N1:].contiguous(),
                                n, a, S1, z1, out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    full = T.direct(x["q64"], x["k64"], x["v64"], n, a)
    check_parity(to_f64(o1), full[:, :, :N1], dtype, say=say, what="first part: ")
    check_parity(to_f64(o2), full[:, :, N1:], dtype, say=say, what="continuation: ")
    Sr, zr = T.state(x["k64"], x["v64"], n)
    assert normwise_rel(to_f64(S2), Sr) < TOL[dtype]
    assert normwise_rel(to_f64(z2)[..., None], zr[..., None]) < TOL[dtype]


def test_empty_inputs():
    d, dv, n = 16, 64, 3
    F = T.n_features(d, n)
    say("empty inputs")
    e = torch.empty((1, 2, 0, d), device="cuda:0")
    ev = torch.empty((1, 2, 0, dv), device="cuda:0")
    S0 = torch.randn((1, 2, F, dv), device="cuda:0")
    z0 = torch.rand((1, 2, F), device="cuda:0")
    o, S, z = tl.prefill(e, e, ev, n, 4.0, S0, z0, return_state=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, dv)
    assert torch.equal(S, S0) and torch.equal(z, z0)
    o, S, z = tl.prefill(e, e, ev, n, 4.0, return_state=True)
    torch.cuda.synchronize()
    assert float(S.abs().max()) == 0.0 and float(z.abs().max()) == 0.0
    eb = torch.empty((0, 2, 10, d), device="cuda:0")
    o = tl.prefill(eb, eb, torch.empty((0, 2, 10, dv), device="cuda:0"), n, 4.0)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 10, dv)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_special_cases(dtype):
    d, dv, N = 16, 64, 300
    x = _inputs(1, 1, N, d, dv, dtype, 33)
    say("special cases", dtype)
    prefix_mean = np.cumsum(x["v64"][0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    # n = 1: prefix mean of v
    o = _run_prefill(x, 1, 4.0, dtype, out_dtype=torch.float32)
    check_parity(to_f64(o)[0, 0][None], prefix_mean[None], dtype, 1, say=say, what="n=1: ")
    # q = 0: prefix mean for any n
    x0 = dict(x)
    x0["q"] = np.zeros_like(x["q"])
    o = _run_prefill(x0, 3, 4.0, dtype, out_dtype=torch.float32)
    check_parity(to_f64(o)[0, 0][None], prefix_mean[None], dtype, 1, say=say, what="q=0: ")
    # constant v: constant output
    xc = dict(x)
    xc["v"] = np.full_like(x["v"], x["v"].flat[0])
    c = float(x["v64"].flat[0])
    o = _run_prefill(xc, 3, 4.0, dtype, out_dtype=torch.float32)
    assert np.max(np.abs(to_f64(o) - c)) < TOL[dtype] * abs(c)


@pytest.mark.parametrize("N", [64, 256])
def test_selectivity_end_to_end(N):
    # posfloor, "The sqrt(N) selectivity tax": a target at the predicted
    # alignment against N-1 distractors at the floor gets weight 0.5.
    d, dv = 16, 16
    t_star = T.required_alignment_based(N, 0.5)
    q = np.zeros((1, 1, N, d), np.float32)
    q[..., 0] = 1
    k = np.zeros((1, 1, N, d), np.float32)
    k[..., 0] = -1
    k[0, 0, 0, 0] = t_star
    v = np.zeros((1, 1, N, dv), np.float32)
    v[0, 0, 0, 0] = 1
    say("selectivity", N)
    o = tl.prefill(to_device(q, "f32"), to_device(k, "f32"), to_device(v, "f32"), 3, 1.0)
    torch.cuda.synchronize()
    got = float(o[0, 0, N - 1, 0])
    ref = T.direct(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64),
                   3, 1.0, rows=[N - 1])[0, 0]
    assert abs(ref - 0.5) < 1e-6  # fp32-rounded t* moves the exact weight a little
    assert abs(got - 0.5) < 1e-4


@pytest.mark.parametrize("d,dv,n", CONFIGS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_after_prefill(d, dv, n, dtype):
    B, H, N, steps = 2, 3, 150, 5
    a = math.sqrt(d)
    x = _inputs(B, H, N + steps, d, dv, dtype, 55, _qk_kind(d, n))
    q, k, v = (to_device(x[s], dtype) for s in "qkv")
    say("decode", d, dv, n, dtype)
    _, S, z = tl.prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous(), n, a,
                         want_output=False, return_state=True)
    outs = []
    for s in range(steps):
        t = N + s
        outs.append(tl.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                              S, z, n, a, out_dtype=torch.float32))
    torch.cuda.synchronize()
    got = np.stack([to_f64(o_) for o_ in outs], axis=2)
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a, rows=list(range(N, N + steps)))
    check_parity(got, ref, dtype, say=say)
    Sr, zr = T.state(x["k64"], x["v64"], n)
    assert normwise_rel(to_f64(S), Sr) < TOL[dtype]


def test_decode_from_oracle_state():
    # decode alone, starting from a state the oracle computed
    d, dv, n, a, N = 16, 64, 3, 4.0, 500
    x = _inputs(1, 4, N + 1, d, dv, "f32", 77)
    S0, z0 = T.state(x["k64"][:, :, :N], x["v64"][:, :, :N], n)
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    say("decode from oracle state")
    o = tl.decode(to_device(x["q"][:, :, N], "f32"), to_device(x["k"][:, :, N], "f32"),
                  to_device(x["v"][:, :, N], "f32"), S, z, n, a)
    torch.cuda.synchronize()
    ref = T.direct(x["q64"], x["k64"], x["v64"], n, a, rows=[N])[:, :, 0]
    check_parity(to_f64(o)[:, :, None], ref[:, :, None], "f32", say=say)


@pytest.mark.parametrize("d,dv,n", [(16, 64, 3), (16, 64, 5)])
def test_prefill_deterministic(d, dv, n):
    x = _inputs(2, 2, 1500, d, dv, "bf16", 91, _qk_kind(d, n))
    say("determinism", d, dv, n)
    o1 = _run_prefill(x, n, 4.0, "bf16")
    o2 = _run_prefill(x, n, 4.0, "bf16")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_bf16_output_matches_fp32_output():
    x = _inputs(1, 2, 333, 16, 64, "bf16", 5)
    say("bf16 vs fp32 output")
    o32 = _run_prefill(x, 3, 4.0, "bf16", out_dtype=torch.float32)
    o16 = _run_prefill(x, 3, 4.0, "bf16", out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))


def test_error_vs_softmax_decreases_with_order():
    # "Expanding Attention", defaults paragraph and the order trade-off: at
    # d=16, dv=64, a=2 with unit-sphere queries and keys, the deviation from
    # causal softmax with the same a falls as terms are added. The kernels'
    # own rounding must stay far below that truncation error, so the GPU
    # error tracks the fp64 oracle's Taylor-vs-softmax error at every n.
    B, H, N, d, dv, a = 1, 2, 1024, 16, 64, 2.0
    x = _inputs(B, H, N, d, dv, "f32", 4242, qk="unit")
    ref = np.stack([T.softmax_causal(x["q64"][0, h], x["k64"][0, h], x["v64"][0, h], a) for h in range(H)])[None]
    errs = []
    for n in (1, 3, 5):
        say("error vs softmax, n =", n)
        o = to_f64(_run_prefill(x, n, a, "f32"))
        tay = T.direct(x["q64"], x["k64"], x["v64"], n, a)
        e_gpu = float(np.max(np.abs(o - ref)))
        e_ora = float(np.max(np.abs(tay - ref)))
        say(f"  n={n}: max|o - softmax| GPU {e_gpu:.3e}, oracle {e_ora:.3e}; normwise GPU "
            f"{normwise_rel(o, ref):.3e}")
        assert abs(e_gpu - e_ora) < 1e-5 + 1e-2 * e_ora
        errs.append(e_gpu)
    assert errs[0] > errs[1] > errs[2]


@pytest.mark.parametrize("d,n", [(16, 3), (32, 3), (16, 5)])
def test_state_rank_on_gpu_features(d, n):
    # "Expanding Attention", "Higher orders": the order-m block of phi has
    # C(d+m-1, m) independent columns, so for N >= F_m generic keys the
    # feature matrix built by the GPU feature map has exactly that rank
    # (singular values cut at 1e-4 of the largest, fp32 features).
    N = 2 * T.n_features(d, n)
    x = _inputs(1, 1, N, d, 4, "f32", 808, qk="unit")
    phi = to_f64(tl.feature_map(to_device(x["k"], "f32")[0, 0], n))
    torch.cuda.synchronize()
    f0 = 0
    for m in range(n):
        Fm = math.comb(d + m - 1, m)
        s = np.linalg.svd(phi[:, f0:f0 + Fm], compute_uv=False)
        rank = int(np.sum(s > 1e-4 * s[0]))
        say(f"d={d} order {m}: rank {rank} of {Fm}")
        assert rank == Fm
        f0 += Fm
    assert f0 == phi.shape[1]


def test_state_truncation_breaks_gpu_readout():
    # "Expanding Attention", "Higher orders": the order-2 state spans all
    # C(d+1, 2) = 136 key directions at d = 16, and none can be dropped. The
    # GPU prefill state is read out through the GPU decode step with orders 0
    # and 1 cleared, so the read-out is the order-2 term alone. Its order-2
    # block is then rebuilt from the GPU feature map's key features truncated
    # to r singular directions: at r = 136 the read-out equals the prefill
    # state's to fp32 rounding, below it the error jumps by orders of magnitude.
    d, dv, n, a, N, M = 16, 64, 3, 4.0, 512, 8
    x = _inputs(1, 1, N, d, dv, "f32", 909, qk="unit")
    k = to_device(x["k"], "f32")
    v = to_device(x["v"], "f32")
    _, S, z = tl.prefill(k, k, v, n, a, want_output=False, return_state=True)
    phi = to_f64(tl.feature_map(k[0, 0].contiguous(), n))
    lo, hi = 1 + d, T.n_features(d, n)
    G = phi[:, lo:hi]
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    assert len(s) == math.comb(d + 1, 2)
    rng = np.random.default_rng(910)
    qm = rng.standard_normal((M, 1, d))
    qm /= np.linalg.norm(qm, axis=-1, keepdims=True)
    qd = torch.tensor(qm, dtype=torch.float32, device="cuda")
    zero_k = torch.zeros((M, 1, d), dtype=torch.float32, device="cuda")
    zero_v = torch.zeros((M, 1, dv), dtype=torch.float32, device="cuda")

    def readout(S2, z2):
        # M copies of the state, orders 0 and 1 cleared; the step's own token
        # (k = 0, v = 0) adds 1 to z_0, so o = a2 phi_2(q) S_2 / (1 + a2 phi_2(q) z_2)
        Sx = torch.zeros((M, 1, hi, dv), dtype=torch.float32, device="cuda")
        zx = torch.zeros((M, 1, hi), dtype=torch.float32, device="cuda")
        Sx[:, :, lo:hi] = S2
        zx[:, :, lo:hi] = z2
        o = tl.decode(qd, zero_k, zero_v, Sx, zx, n, a)
        torch.cuda.synchronize()
        return to_f64(o)[:, 0]

    o_state = readout(S[0, 0, lo:hi], z[0, 0, lo:hi])
    # exact order-2 read-out in fp64 from the same inputs
    w2 = (qm[:, 0] @ x["k64"][0, 0].T / a) ** 2 / 2
    exact = (w2 @ x["v64"][0, 0]) / (1 + w2.sum(axis=1))[:, None]
    say(f"order-2 read-out of the prefill state vs exact: {normwise_rel(o_state, exact, 0):.2e}")
    assert normwise_rel(o_state, exact, 0) < 1e-4
    errs = {}
    for r in (136, 135, 120):
        Gr = (U[:, :r] * s[:r]) @ Vt[:r]
        S2 = torch.tensor(Gr.T @ x["v64"][0, 0], dtype=torch.float32, device="cuda")
        z2 = torch.tensor(Gr.sum(axis=0), dtype=torch.float32, device="cuda")
        errs[r] = normwise_rel(readout(S2, z2), o_state, 0)
        say(f"rank {r} of 136: read-out error {errs[r]:.2e}")
    assert errs[136] < 1e-4
    assert errs[135] > 100 * errs[136] and errs[135] > 1e-2
    assert errs[120] > errs[135]
