"""Shared test helpers: device upload of the seeded inputs and error metrics."""
import numpy as np


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


def sample_rows(N, C=64, extra=64, seed=0):
    """Rows checked at full size: chunk edges, the ends, and a seeded random set."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, C - 1, C, 2 * C - 1, 2 * C, N // 2, N - 2, N - 1}
    rnd = set(rng.choice(N, size=min(extra, N), replace=False).tolist())
    return np.array(sorted(r for r in fixed | rnd if 0 <= r < N))
