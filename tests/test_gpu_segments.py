"""GPU parity of the generic prefill's two-segment plan with a prefix pass
(segment 1 runs segment 0's keys without read-out before its own chunks, no
segment sums), on the eight-wave order-4 kernel with per-token query
features (d = 16, dv = 64, n_terms = 5, bf16): at B=2, H=8, N=2048 the plan
takes two segments (16 heads x 8 feature slices = 128 workgroups per
segment, one per compute unit; tests/test_segplan_host.py checks the cost
model that picks them). Covered: an initial state S0/z0 (continuation after
a first prefill), in place (S = S0, so the final state goes through the
staging area), the decay and the q/k preprocessing, against the fp64 oracle
on the whole sequence ("Expanding Attention": additivity of the states,
closing paragraph).
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

D, DV, NT, A = 16, 64, 5, 4.0
B, H = 2, 8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _part(t, s, e):
    return t[:, :, s:e].contiguous()


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("opts", ["plain", "decay_norm"])
def test_prefix_pass_continuation(inplace, opts):
    # first prefill of N1 tokens, then N2 = 2048 tokens from its state (the
    # two-segment plan); every output row against the oracle on N1 + N2
    N1, N2 = 96, 2048
    kw = {} if opts == "plain" else dict(gamma=0.995, qk_norm=True, q_scale=2.0, k_scale=2.0)
    x = W.make_qkv(B, H, N1 + N2, D, DV, "bf16", 431, "l2x2")
    q, k, v = (to_device(x[s], "bf16") for s in "qkv")
    say("prefix pass continuation", inplace, opts)
    o1, S1, z1 = tl.prefill(_part(q, 0, N1), _part(k, 0, N1), _part(v, 0, N1), NT, A, out_dtype=torch.float32,
                            return_state=True, **kw)
    rest = (_part(q, N1, N1 + N2), _part(k, N1, N1 + N2), _part(v, N1, N1 + N2))
    if inplace:
        o2, S2, z2 = tl.prefill(*rest, NT, A, S1, z1, out_dtype=torch.float32, S=S1, z=z1, **kw)
        assert S2.data_ptr() == S1.data_ptr()
    else:
        o2, S2, z2 = tl.prefill(*rest, NT, A, S1, z1, out_dtype=torch.float32, return_state=True, **kw)
    torch.cuda.synchronize()
    if opts == "plain":
        qp, kp, gamma = x["q64"], x["k64"], 1.0
    else:
        qp, kp, gamma = T.preprocess(x["q64"], True, 2.0), T.preprocess(x["k64"], True, 2.0), 0.995
    full = T.direct(qp, kp, x["v64"], NT, A, gamma=gamma)
    check_parity(to_f64(o1), full[:, :, :N1], "bf16", say=say, what="first part: ")
    check_parity(to_f64(o2), full[:, :, N1:], "bf16", say=say, what="continuation: ")
    # the final state of two heads against a direct sum over every key
    for b, h in ((0, 0), (1, 7)):
        Sr, zr = T.state(kp[b:b + 1, h:h + 1], x["v64"][b:b + 1, h:h + 1], NT, gamma=gamma)
        assert normwise_rel(to_f64(S2[b:b + 1, h:h + 1]), Sr) < TOL["bf16"]
        assert normwise_rel(to_f64(z2[b:b + 1, h:h + 1])[..., None], zr[..., None]) < TOL["bf16"]


def test_prefix_pass_matches_single_segment_rows():
    # the same 2048 tokens as one call and as the first rows of a longer
    # call: a row's output does not depend on how the sequence is split
    N = 2048
    x = W.make_qkv(B, H, N + 64, D, DV, "bf16", 433, "l2x2")
    q, k, v = (to_device(x[s], "bf16") for s in "qkv")
    say("prefix pass vs longer call")
    o_a = tl.prefill(_part(q, 0, N), _part(k, 0, N), _part(v, 0, N), NT, A, out_dtype=torch.float32)
    o_b = tl.prefill(q, k, v, NT, A, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = T.direct(x["q64"][:, :, :N], x["k64"][:, :, :N], x["v64"][:, :, :N], NT, A)
    check_parity(to_f64(o_a), ref, "bf16", say=say, what="N tokens: ")
    check_parity(to_f64(o_b)[:, :, :N], ref, "bf16", say=say, what="first N of N + 64: ")
