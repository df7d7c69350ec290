"""Shared test helpers: device upload of the seeded inputs and error metrics.

Parity is asserted two ways on every output:
  * per head: ||O - O*||_F / ||O*||_F, max over heads, against TOL;
  * per row:  ||o_t - o*_t|| / ||o*_t||, max over every checked row of every
    head, against ROW_TOL, so that an error confined to a few rows (one chunk
    or segment boundary) cannot hide inside a head's norm.
"""
import numpy as np

# per-head bounds: relative error 1e-4 for fp32 inputs, 2e-2 for bf16 inputs
TOL = {"f32": 1e-4, "bf16": 2e-2}
# per-row bounds: every row on its own meets the same bound. Rounding model:
# the bf16 paths round features and the state to bf16 (unit roundoff
# u = 2^-8) and the output to bf16, so a row's relative error is about
# (2 kappa + 1) u for a row condition number kappa of the feature sum; 2e-2 is
# about 5 u and admits kappa up to about 2 (observed worst rows: 5.3e-3 on
# bf16 paths, 1.2e-5 on fp32 paths).
ROW_TOL = dict(TOL)


def to_device(arr, dtype):
    """Seeded storage array (float32, or uint16 bf16 bits) -> torch tensor on cuda:0."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda:0")


def to_f64(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def normwise_rel(o, ref, axis_lead=2):
    """max over heads of ||o - ref||_F / ||ref||_F; arrays shaped [..heads.., rows, dv]."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    lead = o.shape[:axis_lead]
    diff = (o - ref).reshape(int(np.prod(lead)) if lead else 1, -1)
    base = ref.reshape(diff.shape)
    num = np.linalg.norm(diff, axis=1)
    den = np.linalg.norm(base, axis=1)
    return float(np.max(num / den))


def rowwise_rel(o, ref):
    """max over rows (every leading index) of ||o_t - ref_t|| / ||ref_t||
    over the last axis. A NaN anywhere gives NaN. Rows whose reference is
    exactly zero are compared against the largest reference row instead."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(o - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    den = np.where(den > 0, den, max(float(np.max(den)), 1e-300))
    r = num / den
    return float(np.nan) if np.isnan(r).any() else float(np.max(r))


def check_parity(o, ref, dtype, axis_lead=2, say=print, what=""):
    """Assert the per-head and the per-row bound; returns both errors."""
    nw = normwise_rel(o, ref, axis_lead)
    rw = rowwise_rel(o, ref)
    say(f"  {what}normwise {nw:.3e} (bound {TOL[dtype]:g}), worst row {rw:.3e} (bound {ROW_TOL[dtype]:g})")
    assert nw < TOL[dtype], (nw, TOL[dtype])
    assert rw < ROW_TOL[dtype], (rw, ROW_TOL[dtype])
    return nw, rw


def sample_rows(N, C=64, extra=64, seed=0):
    """Rows checked at full size: chunk edges, the ends, and a seeded random set."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, C - 1, C, 2 * C - 1, 2 * C, N // 2, N - 2, N - 1}
    rnd = set(rng.choice(N, size=min(extra, N), replace=False).tolist())
    return np.array(sorted(r for r in fixed | rnd if 0 <= r < N))


def boundary_rows(N, period, every=1, span=2, seed=0, extra=0):
    """Rows around every multiple of `period` (span rows on each side; every
    `every`-th multiple), the first and last rows, and `extra` seeded random
    rows: the positions where chunk and segment bookkeeping can go wrong."""
    s = {0, 1, N - 2, N - 1}
    for b in range(0, N + 1, period * every):
        s.update(range(b - span, b + span))
    if extra:
        rng = np.random.default_rng(seed)
        s.update(rng.choice(N, size=min(extra, N), replace=False).tolist())
    return np.array(sorted(r for r in s if 0 <= r < N))
