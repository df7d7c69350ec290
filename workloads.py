"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and rounds them to the storage type; it
holds none of the attention arithmetic. Recipe, for every workload:

* One PCG64 stream per (batch, head): ``numpy.random.default_rng([seed, b, h])``,
  so any head can be regenerated on its own.
* Draw order inside a head: q [N, d], then k [N, d], then v [N, dv], as
  float64 standard normals.
* ``qk="l2x2"``: every q and k row is scaled to Euclidean norm 2 in float64
  before rounding (the order-4 workload); ``qk="unit"``: to norm 1 (the
  unit-sphere defaults of the accuracy-against-softmax measurement).
* Rounding: float64 -> float32 (round to nearest even) -> bf16 (round to
  nearest even on the fp32 bit pattern) when the storage type is bf16.

The returned float64 arrays hold exactly the rounded values, so a float64
reference computes on the very numbers the device sees.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_THREADS = min(16, os.cpu_count() or 1)


def _pmap(fn, items):
    """Map over heads in a thread pool (the draws are per-head seeded, so the
    result does not depend on the pool)."""
    items = list(items)
    if len(items) < 8:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(_THREADS) as ex:
        return list(ex.map(fn, items))


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dv: int
    n_terms: int
    a: float
    dtype: str          # "f32" or "bf16": storage type of q, k, v
    seed: int
    qk: str = "normal"  # "normal", "l2x2" or "unit"
    steps: int = 0      # decode steps after an N-token prefill (decode workload)
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "order2_tiny_fp32": Workload(
        "order2_tiny_fp32", B=1, H=1, N=256, d=16, dv=16, n_terms=3, a=4.0,
        dtype="f32", seed=1001,
        notes="order 2, t = q.k/sqrt(d), fp32 parity case"),
    "based_order2_prefill": Workload(
        "based_order2_prefill", B=4, H=16, N=4096, d=16, dv=64, n_terms=3, a=4.0,
        dtype="bf16", seed=1002,
        notes="Based-style order-2 prefill, 153 features, bf16 in, fp32 accumulate"),
    "order4_prefill": Workload(
        "order4_prefill", B=2, H=8, N=8192, d=16, dv=64, n_terms=5, a=4.0,
        dtype="bf16", seed=1003, qk="l2x2",
        notes="order 4, 4845 features, q/k rows at norm 2"),
    "order2_decode": Workload(
        "order2_decode", B=64, H=16, N=32768, d=16, dv=64, n_terms=3, a=4.0,
        dtype="f32", seed=1004, steps=1024,
        notes="states from a 32768-token fp32 prefill, then 1024 decode steps"),
    "long_order2_prefill": Workload(
        "long_order2_prefill", B=1, H=8, N=65536, d=64, dv=64, n_terms=3, a=8.0,
        dtype="bf16", seed=1005,
        notes="long-context order 2, d=64, 2145 features"),
}


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to(x64: np.ndarray, dtype: str):
    """Round float64 data to the storage type.

    Returns (stored, exact64): ``stored`` is float32 or uint16 bf16 bits,
    ``exact64`` the same values as float64.
    """
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "bf16":
        bits = bf16_bits(x32)
        return bits, bf16_to_f64(bits)
    raise ValueError(dtype)


def _head_draw(seed, b, h, N, d, dv, qk):
    rng = np.random.default_rng([seed, b, h])
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, dv))
    if qk in ("l2x2", "unit"):
        r = 2.0 if qk == "l2x2" else 1.0
        q = r * q / np.linalg.norm(q, axis=1, keepdims=True)
        k = r * k / np.linalg.norm(k, axis=1, keepdims=True)
    return q, k, v


def make_qkv(B, H, N, d, dv, dtype="f32", seed=0, qk="normal", heads=None):
    """Seeded q, k, v in layout [B, H, N, .].

    Returns dict with 'q', 'k', 'v' (storage arrays: float32, or uint16 bf16
    bits) and 'q64', 'k64', 'v64' (the same values in float64). With
    ``heads`` (list of (b, h)) only those heads are drawn and the arrays
    have shape [len(heads), N, .].
    """
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    shp = (B, H) if heads is None else (len(sel),)
    out = {}
    draws = _pmap(lambda bh: _head_draw(seed, bh[0], bh[1], N, d, dv, qk), sel)
    for j, (name, w) in enumerate((("q", d), ("k", d), ("v", dv))):
        x = np.stack([t[j] for t in draws]).reshape(shp + (N, w)) if sel else np.zeros(shp + (N, w))
        stored, exact = round_to(x, dtype)
        out[name] = stored
        out[name + "64"] = exact
    return out


def make_workload(w: Workload, heads=None, N=None):
    """Inputs of a named workload (optionally a subset of heads or a shorter N).

    A shorter N is a prefix of the full-length draw only for N == w.N; other
    N values make a fresh draw of that length from the same per-head seed.
    """
    return make_qkv(w.B, w.H, w.N if N is None else N, w.d, w.dv, w.dtype,
                    w.seed, w.qk, heads)


def make_decode_inputs(w: Workload, heads=None, steps=None):
    """Decode workload: per head, a prefill of N tokens (k, v only), then
    ``steps`` single-token (q, k, v) draws. Same per-head stream layout:
    prefill k [N, d], prefill v [N, dv], then for the steps q [S, d], k [S, d],
    v [S, dv]. All float32 (the workload is fp32).
    """
    S = w.steps if steps is None else steps
    sel = [(b, h) for b in range(w.B) for h in range(w.H)] if heads is None else list(heads)
    shp = (w.B, w.H) if heads is None else (len(sel),)
    pk = np.empty((len(sel), w.N, w.d), np.float32)
    pv = np.empty((len(sel), w.N, w.dv), np.float32)
    sq = np.empty((len(sel), S, w.d), np.float32)
    sk = np.empty((len(sel), S, w.d), np.float32)
    sv = np.empty((len(sel), S, w.dv), np.float32)

    def one(i):
        b, h = sel[i]
        rng = np.random.default_rng([w.seed, b, h])
        pk[i] = rng.standard_normal((w.N, w.d))
        pv[i] = rng.standard_normal((w.N, w.dv))
        sq[i] = rng.standard_normal((S, w.d))
        sk[i] = rng.standard_normal((S, w.d))
        sv[i] = rng.standard_normal((S, w.dv))

    _pmap(one, range(len(sel)))
    r = lambda x: x.reshape(shp + x.shape[1:])
    return {"prefill_k": r(pk), "prefill_v": r(pv),
            "step_q": r(sq), "step_k": r(sk), "step_v": r(sv)}
