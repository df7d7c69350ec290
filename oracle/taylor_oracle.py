"""Plain fp64 CPU oracle for causal Taylor-series linear attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports, calls or links it,
and this module imports nothing from the product path.

Everything here is written from the definitions on the source pages, slowly
and visibly, in float64 (or exact ``fractions.Fraction``):

* "Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
  with a Fixed Number of Recurrent States" (called EA below): the truncated
  expansion of exp(q.k/a) with coefficients 1/(m! a^m), the tensor-power
  identity, the symmetric basis of width C(d+m-1, m) ("Higher orders"), the
  per-order states ("Memory"), the causal mask and normalisation against
  softmax with the same a (the defaults paragraph), exactness and
  additivity of the recursion (closing paragraph).
* "posfloor" README (called PF below): the order-2 map
  [1, x, (x outer x)/sqrt 2] and its weight 1 + t + t^2/2; the 1/2 floor and
  the even-order minima ("The 1/2 positivity floor"); the required-alignment
  law and the end-to-end weight check ("The sqrt(N) selectivity tax").
* The Spanish linear-attention explainer (called LA below): the recurrence
  S_t = S_{t-1} + v_t phi(k_t)^T, o_t = S_t phi(q_t) -- update first, then
  read out; and, in its paragraph on superposed memory, forgetting by a decay
  that multiplies S_{t-1} before the write (the Mamba-2 reading of linear
  attention with decay).

Readings taken where the pages leave a step open:
* n_terms counts Taylor terms m = 0 .. n-1; "order k" means n = k + 1.
* Output is normalised by the same weights (EA compares against softmax).
* The causal mask is inclusive (s <= t), matching LA's update-then-read.
* phi_m carries only the sqrt-multinomial weights; alpha_m = 1/(m! a^m) is
  applied at read-out (or folded into phi(q) when ``a`` is passed to phi).
* Canonical feature order: m ascending; within an order, non-decreasing
  index tuples in lexicographic order.
* Query/key preprocessing (``preprocess``): EA treats unit-sphere rows as
  mandatory and cites per-head temperatures; the reading taken divides each
  row by its l2 norm (a zero row stays zero), then multiplies queries by a
  scale and a per-head factor and keys by a scale. The method then runs on
  the preprocessed rows.
* Decay (``gamma``): one constant factor gamma in (0, 1] for every step,
  applied to S and z alike (z is the state of the all-ones value column), so
  the output stays a normalised average: token s enters the output at time
  t >= s with weight gamma^(t-s) w_ts, and an initial state S0/z0 (the state
  just before token 0) with gamma^(t+1). gamma = 1 is the plain method.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np

__all__ = [
    "n_features", "monomials", "multinomial", "taylor_weight", "phi",
    "direct", "state", "recurrent", "decode_step", "exact_fraction",
    "softmax_causal", "truncated_exp_minimum", "required_alignment_based",
    "required_alignment_softmax",
]


# --------------------------------------------------------------------------
# Basis (EA "Higher orders": minimal symmetric basis of width C(d+m-1, m))
# --------------------------------------------------------------------------

def n_features(d: int, n_terms: int) -> int:
    """Total width sum_{m<n} C(d+m-1, m) of the symmetric basis (EA "Memory")."""
    return sum(math.comb(d + m - 1, m) for m in range(n_terms))


def monomials(d: int, m: int) -> list[tuple[int, ...]]:
    """Index tuples i_1 <= ... <= i_m over {0..d-1}, lexicographic order.

    Each tuple is one monomial prod_j x[i_j] of degree m; there are
    C(d+m-1, m) of them (EA "Higher orders").
    """
    return list(itertools.combinations_with_replacement(range(d), m))


def multinomial(tup: tuple[int, ...]) -> int:
    """m! / prod_i c_i! where c_i counts index i in the tuple.

    This is the number of ordered index sequences that sort to ``tup``: the
    multiplicity of the monomial in the tensor power x^{(x)m}, so the
    symmetric feature needs weight sqrt(multinomial) for
    phi_m(x).phi_m(y) = (x.y)^m (multinomial theorem).
    """
    counts: dict[int, int] = {}
    for i in tup:
        counts[i] = counts.get(i, 0) + 1
    den = 1
    for c in counts.values():
        den *= math.factorial(c)
    return math.factorial(len(tup)) // den


# --------------------------------------------------------------------------
# Weight function (EA: exp(t) ~ sum_{m<n} t^m / m!, t = q.k / a)
# --------------------------------------------------------------------------

def taylor_weight(t, n_terms: int):
    """w_n(t) = sum_{m=0}^{n-1} t^m / m!, evaluated term by term.

    ``t`` may be a float, an ndarray or a Fraction.
    """
    total = 0 * t
    power = 1 + 0 * t
    for m in range(n_terms):
        total = total + power / math.factorial(m)
        power = power * t
    return total


# --------------------------------------------------------------------------
# Feature map (EA tensor-power identity + symmetric basis)
# --------------------------------------------------------------------------

def phi(x, n_terms: int, a: float | None = None) -> np.ndarray:
    """Symmetric feature map, rows x d -> rows x F, float64.

    Block m (m = 0..n-1) holds sqrt(multinomial(tup)) * prod_j x[:, tup_j]
    for every tuple of ``monomials(d, m)``. With ``a`` given, block m is also
    scaled by sqrt(alpha_m) = (m! a^m)^(-1/2), so that phi(x).phi(y) equals
    w_n(x.y / a).
    """
    x = np.asarray(x, dtype=np.float64)
    rows, d = x.shape
    cols = []
    for m in range(n_terms):
        scale = 1.0 if a is None else 1.0 / math.sqrt(math.factorial(m) * a ** m)
        for tup in monomials(d, m):
            col = np.ones(rows, dtype=np.float64)
            for i in tup:
                col = col * x[:, i]
            cols.append(col * math.sqrt(multinomial(tup)) * scale)
    return np.stack(cols, axis=1)


def alpha_vector(d: int, n_terms: int, a: float) -> np.ndarray:
    """alpha_m = 1/(m! a^m) repeated over the C(d+m-1, m) features of order m."""
    out = []
    for m in range(n_terms):
        out += [1.0 / (math.factorial(m) * a ** m)] * math.comb(d + m - 1, m)
    return np.array(out, dtype=np.float64)


# --------------------------------------------------------------------------
# Direct causal form (the definition)
# --------------------------------------------------------------------------

def direct(q, k, v, n_terms: int, a: float, S0=None, z0=None,
           rows=None, block: int = 256, gamma: float = 1.0) -> np.ndarray:
    """Causal normalised polynomial-weighted average, O(N^2), float64.

    For one head (q, k: N x d, v: N x dv):
        w_ts = w_n(q_t.k_s / a) for s <= t,
        o_t  = sum_{s<=t} w_ts v_s / sum_{s<=t} w_ts.
    With an initial state (S0: F x dv, z0: F), the earlier tokens that the
    state summarises add alpha-weighted phi(q_t).S0 and phi(q_t).z0 to the
    numerator and denominator (state additivity, EA closing paragraph).

    Leading batch axes are allowed: q[..., N, d]. ``rows`` restricts the
    output to the given query positions (the result is then [..., len(rows), dv]).
    With a decay gamma < 1 every weight w_ts is multiplied by gamma^(t-s) and
    the initial-state terms by gamma^(t+1) (module notes).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim > 2:
        lead = q.shape[:-2]
        out = None
        for idx in np.ndindex(*lead):
            s0 = None if S0 is None else np.asarray(S0)[idx]
            zz = None if z0 is None else np.asarray(z0)[idx]
            o = direct(q[idx], k[idx], v[idx], n_terms, a, s0, zz, rows, block, gamma)
            if out is None:
                out = np.empty(lead + o.shape, dtype=np.float64)
            out[idx] = o
        return out
    N = q.shape[0]
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(sel), v.shape[1]), dtype=np.float64)
    for b0 in range(0, len(sel), block):
        r = sel[b0:b0 + block]
        e = int(r.max()) + 1
        T = (q[r] @ k[:e].T) / a
        W = taylor_weight(T, n_terms)
        W = np.where(np.arange(e)[None, :] <= r[:, None], W, 0.0)
        if gamma != 1.0:
            lag = np.maximum(r[:, None] - np.arange(e)[None, :], 0).astype(np.float64)
            W = W * np.power(float(gamma), lag)
        num = W @ v[:e]
        den = W.sum(axis=1)
        if S0 is not None:
            fq = phi(q[r], n_terms) * alpha_vector(q.shape[1], n_terms, a)
            carry = np.power(float(gamma), r + 1.0) if gamma != 1.0 else np.ones(len(r))
            num = num + carry[:, None] * (fq @ np.asarray(S0, dtype=np.float64))
            den = den + carry * (fq @ np.asarray(z0, dtype=np.float64))
        out[b0:b0 + len(r)] = num / den[:, None]
    return out


# --------------------------------------------------------------------------
# States (EA "Memory"; LA recurrence)
# --------------------------------------------------------------------------

def state(k, v, n_terms: int, S0=None, z0=None, gamma: float = 1.0):
    """Per-order states after the given tokens: S = S0 + phi(K)^T V, z = z0 + phi(K)^T 1.

    With a decay, token s of N enters with gamma^(N-1-s) and S0, z0 with gamma^N.
    Shapes: k [..., N, d], v [..., N, dv] -> S [..., F, dv], z [..., F].
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.ndim > 2:
        lead = k.shape[:-2]
        F = n_features(k.shape[-1], n_terms)
        S = np.empty(lead + (F, v.shape[-1]))
        z = np.empty(lead + (F,))
        for idx in np.ndindex(*lead):
            S[idx], z[idx] = state(k[idx], v[idx], n_terms,
                                   None if S0 is None else np.asarray(S0)[idx],
                                   None if z0 is None else np.asarray(z0)[idx], gamma)
        return S, z
    fk = phi(k, n_terms)
    N = k.shape[0]
    dec = np.power(float(gamma), np.arange(N - 1, -1, -1, dtype=np.float64)) if gamma != 1.0 else np.ones(N)
    S = (fk * dec[:, None]).T @ v
    z = fk.T @ dec
    if S0 is not None:
        carry = float(gamma) ** N if gamma != 1.0 else 1.0
        S = S + carry * np.asarray(S0, dtype=np.float64)
        z = z + carry * np.asarray(z0, dtype=np.float64)
    return S, z


def recurrent(q, k, v, n_terms: int, a: float, S0=None, z0=None, gamma: float = 1.0):
    """Token-by-token recurrence for one head (LA: update, then read out).

    S_t = gamma S_{t-1} + phi(k_t) v_t^T,  z_t = gamma z_{t-1} + phi(k_t),
    o_t = sum_m alpha_m phi_m(q_t).S_m,t / sum_m alpha_m phi_m(q_t).z_m,t.
    Returns (o [N, dv], S [F, dv], z [F]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    F = n_features(d, n_terms)
    S = np.zeros((F, v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64)
    z = np.zeros(F) if z0 is None else np.array(z0, dtype=np.float64)
    alpha = alpha_vector(d, n_terms, a)
    out = np.empty((N, v.shape[1]))
    for t in range(N):
        fk = phi(k[t:t + 1], n_terms)[0]
        S = gamma * S + np.outer(fk, v[t])
        z = gamma * z + fk
        fq = phi(q[t:t + 1], n_terms)[0] * alpha
        out[t] = (fq @ S) / (fq @ z)
    return out, S, z


def decode_step(q, k, v, S, z, n_terms: int, a: float, gamma: float = 1.0):
    """One generation step for one head: decay, update with (k, v), then read out with q.

    Returns (o [dv], S_new [F, dv], z_new [F]).
    """
    fk = phi(np.asarray(k, dtype=np.float64)[None, :], n_terms)[0]
    S_new = gamma * np.asarray(S, dtype=np.float64) + np.outer(fk, np.asarray(v, dtype=np.float64))
    z_new = gamma * np.asarray(z, dtype=np.float64) + fk
    d = len(q)
    fq = phi(np.asarray(q, dtype=np.float64)[None, :], n_terms)[0] * alpha_vector(d, n_terms, a)
    return (fq @ S_new) / (fq @ z_new), S_new, z_new


# --------------------------------------------------------------------------
# Exact rational evaluation (tiny inputs)
# --------------------------------------------------------------------------

def exact_fraction(q, k, v, n_terms: int, a) -> list[list[Fraction]]:
    """The direct form in exact rational arithmetic; inputs must be rationals.

    Pure-Python loops; meant for N, d, dv of a few.
    """
    a = Fraction(a)
    q = [[Fraction(x) for x in row] for row in q]
    k = [[Fraction(x) for x in row] for row in k]
    v = [[Fraction(x) for x in row] for row in v]
    out = []
    for t in range(len(q)):
        num = [Fraction(0)] * len(v[0])
        den = Fraction(0)
        for s in range(t + 1):
            dot = sum((qi * ki for qi, ki in zip(q[t], k[s])), Fraction(0))
            w = taylor_weight(dot / a, n_terms)
            den += w
            num = [nu + w * vj for nu, vj in zip(num, v[s])]
        out.append([nu / den for nu in num])
    return out


# --------------------------------------------------------------------------
# Query/key preprocessing (EA: rows on the unit sphere; per-head temperature)
# --------------------------------------------------------------------------

def preprocess(x, normalise: bool = True, scale: float = 1.0, head_scale=None) -> np.ndarray:
    """Rows of x [..., H, N, d] (or [N, d]) divided by their l2 norm (zero rows
    stay zero), times ``scale`` and, per head, ``head_scale[h]`` (x[..., h, :, :])."""
    x = np.asarray(x, dtype=np.float64)
    if normalise:
        n = np.linalg.norm(x, axis=-1, keepdims=True)
        x = np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    x = x * float(scale)
    if head_scale is not None:
        hs = np.asarray(head_scale, dtype=np.float64)
        x = x * hs.reshape(hs.shape + (1, 1))
    return x


# --------------------------------------------------------------------------
# Causal softmax with the same scale (EA's reference outputs)
# --------------------------------------------------------------------------

def softmax_causal(q, k, v, a: float, block: int = 256) -> np.ndarray:
    """Causally masked softmax attention exp(q.k / a), one head, float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N = q.shape[0]
    out = np.empty((N, v.shape[1]))
    for r0 in range(0, N, block):
        r = np.arange(r0, min(N, r0 + block))
        e = int(r[-1]) + 1
        T = (q[r] @ k[:e].T) / a
        T = np.where(np.arange(e)[None, :] <= r[:, None], T, -np.inf)
        T = T - T.max(axis=1, keepdims=True)
        W = np.exp(T)
        out[r0:r0 + len(r)] = (W @ v[:e]) / W.sum(axis=1)[:, None]
    return out


# --------------------------------------------------------------------------
# posfloor facts ("The 1/2 positivity floor", "The sqrt(N) selectivity tax")
# --------------------------------------------------------------------------

def truncated_exp_minimum(order: int) -> tuple[float, float]:
    """Global minimum (t_min, w_min) of sum_{m<=order} t^m/m! for even order.

    The derivative of the degree-``order`` partial sum is the degree
    ``order-1`` partial sum, so the minimiser is that polynomial's real root.
    """
    if order % 2:
        raise ValueError("odd truncations are unbounded below")
    if order == 0:
        return 0.0, 1.0
    coeffs = [1.0 / math.factorial(m) for m in range(order - 1, -1, -1)]
    roots = np.roots(coeffs)
    real = [r.real for r in roots if abs(r.imag) < 1e-9]
    t_min = min(real, key=lambda t: taylor_weight(t, order + 1))
    return t_min, taylor_weight(t_min, order + 1)


def required_alignment_based(N: int, w: float, distractor_t: float = -1.0) -> float:
    """Alignment t a target key needs under 1 + t + t^2/2 to get normalised weight w.

    The N - 1 distractors all sit at alignment ``distractor_t`` (the floor,
    t = -1, by default). Their summed weight is (N-1) w_3(distractor_t); the
    target needs unnormalised weight W = w (N-1) w_3(distractor_t) / (1 - w),
    and the larger root of 1 + t + t^2/2 = W is returned.
    """
    W = w * (N - 1) * taylor_weight(distractor_t, 3) / (1.0 - w)
    # t^2/2 + t + (1 - W) = 0  ->  t = -1 + sqrt(1 - 2 (1 - W))
    return -1.0 + math.sqrt(1.0 - 2.0 * (1.0 - W))


def required_alignment_softmax(N: int, w: float) -> float:
    """Alignment softmax needs for weight w when N - 1 distractors go to weight ~0.

    With distractor scores at 0 (weight e^0 = 1 each) exp(t) = w (N-1)/(1-w).
    """
    return math.log(w * (N - 1) / (1.0 - w))
