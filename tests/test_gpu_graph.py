"""HIP graph capture of the path: prefill (all three kernel families) and
decode steps captured once and replayed several times, with eager work and
synchronisations between the replays; every replay must reproduce the eager
results bit for bit (the kernels are deterministic and the library records no
memset nodes: the prefill's flag reset is a kernel of its own)."""
import sys

import pytest

import workloads as W
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("needs a GPU", allow_module_level=True)

import taylor_series_linear_amd as tl  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# (B, H, N, d, dv, n_terms, a, dtype): the order-2 d=16 bf16 single-pass kernel
# (several segments per head), the generic kernel (order 4), the d=64 kernel
CASES = [(2, 8, 2048, 16, 64, 3, 4.0, "bf16"), (1, 2, 700, 16, 64, 5, 4.0, "bf16"),
         (1, 2, 1500, 64, 64, 3, 8.0, "bf16")]
STEPS = 3


def _inputs():
    xs = []
    for i, (B, H, N, d, dv, n, a, dt) in enumerate(CASES):
        x = W.make_qkv(B, H, N, d, dv, dt, 7100 + i)
        q, k, v = (to_device(x[s], dt) for s in "qkv")
        s = W.make_qkv(STEPS, B * H, 1, d, dv, "f32", 7200 + i)
        dq, dk, dvv = (to_device(s[c], "f32").view(STEPS, B, H, -1) for c in "qkv")
        xs.append((q, k, v, dq, dk, dvv))
    return xs


def _run(xs, bufs):
    """The captured sequence: per case a prefill with output, a prefill that
    writes the state, then STEPS decode steps on that state (fp32 inputs)."""
    for (B, H, N, d, dv, n, a, dt), (q, k, v, dq, dk, dvv), b in zip(CASES, xs, bufs):
        b["o"] = tl.prefill(q, k, v, n, a, workspace=b["ws"])
        tl.prefill(q, k, v, n, a, want_output=False, S=b["S"], z=b["z"], workspace=b["ws"])
        for t in range(STEPS):
            tl.decode(dq[t], dk[t], dvv[t], b["S"], b["z"], n, a, o=b["od"][t])


def _bufs():
    out = []
    for (B, H, N, d, dv, n, a, dt) in CASES:
        F = tl.feature_dim(d, n)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        ws = tl.prefill_workspace_bytes(B, H, N, d, dv, n, tdt)
        out.append({
            "S": torch.zeros((B, H, F, dv), dtype=torch.float32, device="cuda"),
            "z": torch.zeros((B, H, F), dtype=torch.float32, device="cuda"),
            "od": torch.zeros((STEPS, B, H, dv), dtype=torch.float32, device="cuda"),
            "ws": torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda"),
        })
    return out


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_graph_replays_match_eager():
    xs = _inputs()
    say("graph: eager reference")
    ref = _bufs()
    _run(xs, ref)
    torch.cuda.synchronize()

    bufs = _bufs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(xs, bufs)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph: capture")
    with torch.cuda.graph(g):
        _run(xs, bufs)
    torch.cuda.synchronize()
    for rep in range(4):
        for b in bufs:
            for t in b.values():
                if t.dtype != torch.uint8:
                    t.fill_(7)   # stale values that a skipped write would expose
        g.replay()
        torch.cuda.synchronize()
        say(f"graph: replay {rep}")
        for i, (b, r) in enumerate(zip(bufs, ref)):
            for name in ("o", "S", "z", "od"):
                assert _same(b[name], r[name]), f"case {CASES[i]}, {name}, replay {rep}"
        # eager work between replays, on the same buffers' neighbours
        other = _bufs()
        _run(xs, other)
        torch.cuda.synchronize()
        assert _same(other[0]["o"], ref[0]["o"])
