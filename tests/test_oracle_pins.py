"""Pins for the fp64 oracle: facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: printed
values (tests/golden/), closed forms, brute force, exact rational arithmetic
or invariants. CPU only.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import taylor_oracle as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


# ----------------------------------------------------------------------------
# Feature map: multinomial theorem and tensor-power identity (C-P1)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,m", [(1, 3), (3, 2), (4, 3), (5, 4), (16, 2), (16, 4), (64, 2), (3, 6), (4, 5),
                                 (16, 6)])
def test_phi_block_dot_is_power_of_dot(d, m):
    rng = np.random.default_rng(d * 10 + m)
    x = rng.standard_normal((7, d))
    y = rng.standard_normal((5, d))
    F_lo = T.n_features(d, m)
    F_hi = T.n_features(d, m + 1)
    px = T.phi(x, m + 1)[:, F_lo:F_hi]
    py = T.phi(y, m + 1)[:, F_lo:F_hi]
    want = (x @ y.T) ** m
    assert np.max(np.abs(px @ py.T - want)) <= 1e-12 * np.max(np.abs(want)) + 1e-300


@pytest.mark.parametrize("d,m", [(2, 2), (3, 3), (4, 2), (3, 4), (2, 6), (3, 5)])
def test_phi_matches_full_tensor_power(d, m):
    # <x^{(x)m}, y^{(x)m}> built from explicit Kronecker powers.
    rng = np.random.default_rng(99 + d + m)
    x, y = rng.standard_normal(d), rng.standard_normal(d)
    kx, ky = np.ones(1), np.ones(1)
    for _ in range(m):
        kx, ky = np.kron(kx, x), np.kron(ky, y)
    lo, hi = T.n_features(d, m), T.n_features(d, m + 1)
    px = T.phi(x[None], m + 1)[0, lo:hi]
    py = T.phi(y[None], m + 1)[0, lo:hi]
    assert abs(px @ py - kx @ ky) <= 1e-12 * abs(kx @ ky)
    # The sqrt-multinomial weight squared counts the ordered index sequences
    # that sort to the tuple (the coordinates of x^{(x)m} it stands for).
    for tup in T.monomials(d, m):
        count = sum(1 for idx in itertools.product(range(d), repeat=m)
                    if tuple(sorted(idx)) == tup)
        assert count == T.multinomial(tup)


def test_based_order2_identity():
    # PF: phi(x) = [1, x, (x outer x)/sqrt 2] gives phi(q).phi(k) = 1 + t + t^2/2.
    rng = np.random.default_rng(7)
    d, a = 16, 4.0
    q = rng.standard_normal((6, d))
    k = rng.standard_normal((9, d))

    def based(x):
        x = x / math.sqrt(a)  # t = q.k / a
        outer = np.einsum("ri,rj->rij", x, x).reshape(len(x), -1) / math.sqrt(2.0)
        return np.concatenate([np.ones((len(x), 1)), x, outer], axis=1)

    t = q @ k.T / a
    closed = 1 + t + t ** 2 / 2
    ours = T.phi(q, 3, a=a) @ T.phi(k, 3, a=a).T
    assert np.max(np.abs(based(q) @ based(k).T - closed)) < 1e-12 * np.max(np.abs(closed))
    assert np.max(np.abs(ours - closed)) < 1e-12 * np.max(np.abs(closed))
    # Deduplicated width 1 + d + d(d+1)/2 against Based's 1 + d + d^2.
    assert T.phi(q, 3).shape[1] == 1 + d + d * (d + 1) // 2 == 153


def test_alpha_folding_gives_truncated_exp():
    rng = np.random.default_rng(11)
    for d, n, a in [(16, 5, 4.0), (64, 3, 8.0), (3, 7, 2.0)]:
        q = rng.standard_normal((4, d))
        k = rng.standard_normal((4, d))
        t = q @ k.T / a
        closed = sum(t ** m / math.factorial(m) for m in range(n))
        got = T.phi(q, n, a=a) @ T.phi(k, n, a=a).T
        assert np.max(np.abs(got - closed)) < 1e-12 * np.max(np.abs(closed))
        got2 = (T.phi(q, n) * T.alpha_vector(d, n, a)) @ T.phi(k, n).T
        assert np.max(np.abs(got2 - closed)) < 1e-12 * np.max(np.abs(closed))


def test_feature_order_is_canonical():
    # m ascending, then non-decreasing tuples in lexicographic order.
    d = 3
    tuples = [t for m in range(4) for t in T.monomials(d, m)]
    assert tuples[:5] == [(), (0,), (1,), (2,), (0, 0)]
    for m in range(4):
        blk = T.monomials(d, m)
        assert blk == sorted(blk)
        assert all(list(t) == sorted(t) for t in blk)
    x = np.array([[2.0, 3.0, 5.0]])
    f = T.phi(x, 3)[0]
    # [1, x0, x1, x2, x0^2, sqrt2 x0x1, sqrt2 x0x2, x1^2, sqrt2 x1x2, x2^2]
    want = [1, 2, 3, 5, 4, math.sqrt(2) * 6, math.sqrt(2) * 10, 9, math.sqrt(2) * 15, 25]
    assert np.allclose(f, want, rtol=1e-15, atol=0)


# ----------------------------------------------------------------------------
# Widths (C-P2)
# ----------------------------------------------------------------------------

def test_widths():
    g = gold("expanding_attention_facts.json")
    for row in g["widths"]:
        d, n, F = row["d"], row["n_terms"], row["F"]
        assert T.n_features(d, n) == F
        assert math.comb(d + n - 1, n - 1) == F  # hockey-stick closed form
        assert T.phi(np.ones((1, d)), n).shape[1] == F
    # order 6 at d = 16 (the highest even order of the positivity-floor
    # README's minima): the width by brute-force enumeration of the basis
    F6 = sum(sum(1 for _ in itertools.combinations_with_replacement(range(16), m)) for m in range(7))
    assert F6 == T.n_features(16, 7) == math.comb(22, 6) == 74613
    cap = gold("posfloor_printed.json")["gram_capacity"]
    d = cap["d"]
    assert (d + 1) * (d + 2) // 2 == cap["value"] == T.n_features(d, 3)


# ----------------------------------------------------------------------------
# State rank law (C-P3)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("case", gold("expanding_attention_facts.json")["rank_cases"])
def test_state_rank(case):
    d, m, r = case["d"], case["m"], case["rank"]
    assert math.comb(d + m - 1, m) == r
    rng = np.random.default_rng(5)
    N = 3 * r
    K = rng.standard_normal((N, d))
    lo, hi = T.n_features(d, m), T.n_features(d, m + 1)
    Phi = T.phi(K, m + 1)[:, lo:hi]
    s = np.linalg.svd(Phi, compute_uv=False)
    assert int(np.sum(s > s[0] * 1e-10)) == r
    if d ** m <= 4096:
        def tpow(x):
            out = np.ones(1)
            for _ in range(m):
                out = np.kron(out, x)
            return out
        tp = np.stack([tpow(kk) for kk in K])
        s2 = np.linalg.svd(tp, compute_uv=False)
        assert int(np.sum(s2 > s2[0] * 1e-10)) == r


@pytest.mark.parametrize("d,m", [(3, 6), (4, 5), (2, 6)])
def test_state_rank_high_orders(d, m):
    # "Higher orders": the rank of the order-m key features (and of the full
    # tensor power) is C(d+m-1, m), for the orders 5 and 6 as well
    r = math.comb(d + m - 1, m)
    rng = np.random.default_rng(17 + d + m)
    K = rng.standard_normal((3 * r, d))
    lo, hi = T.n_features(d, m), T.n_features(d, m + 1)
    s = np.linalg.svd(T.phi(K, m + 1)[:, lo:hi], compute_uv=False)
    assert hi - lo == r and int(np.sum(s > s[0] * 1e-10)) == r

    def tpow(x):
        out = np.ones(1)
        for _ in range(m):
            out = np.kron(out, x)
        return out
    s2 = np.linalg.svd(np.stack([tpow(kk) for kk in K]), compute_uv=False)
    assert int(np.sum(s2 > s2[0] * 1e-10)) == r


def test_rank_truncation_breaks_readout():
    # Truncating the order-m state below C(d+m-1, m) makes the read-out O(1) wrong.
    d, m, dv = 4, 2, 8
    r = math.comb(d + m - 1, m)
    rng = np.random.default_rng(8)
    K = rng.standard_normal((200, d))
    V = rng.standard_normal((200, dv))
    Q = rng.standard_normal((50, d))
    lo, hi = T.n_features(d, m), T.n_features(d, m + 1)
    S = T.phi(K, m + 1)[:, lo:hi].T @ V
    fq = T.phi(Q, m + 1)[:, lo:hi]
    exact = ((Q @ K.T) ** m) @ V
    full = fq @ S
    assert rel(full, exact) < 1e-12
    # S is F_m x dv with dv < F_m here; use the key-side Gram instead:
    G = T.phi(K, m + 1)[:, lo:hi]
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    assert len(s) == r
    for keep in (r - 1, r - 3):
        Gt = (U[:, :keep] * s[:keep]) @ Vt[:keep]
        approx = fq @ (Gt.T @ V)
        assert rel(approx, exact) > 1e-3
    Gt = (U[:, :r] * s[:r]) @ Vt[:r]
    assert rel(fq @ (Gt.T @ V), exact) < 1e-12


# ----------------------------------------------------------------------------
# posfloor facts (C-P4 .. C-P8)
# ----------------------------------------------------------------------------

def test_order2_floor():
    g = gold("posfloor_printed.json")["order2_floor"]
    assert T.taylor_weight(Fraction(-1), 3) == Fraction(1, 2) == Fraction(g["value"])
    t = np.linspace(-50, 50, 200001)
    w = T.taylor_weight(t, 3)
    assert w.min() >= 0.5
    assert abs(t[np.argmin(w)] - g["at_t"]) < 1e-3


def test_even_minima_and_odd_roots():
    g = gold("posfloor_printed.json")["even_minima"]
    for order, printed in zip(g["orders"], g["values"]):
        t_min, w_min = T.truncated_exp_minimum(order)
        assert round(w_min, g["decimals"]) == printed
        # min value equals t*^order / order! (the lower partial sum vanishes there)
        assert math.isclose(w_min, t_min ** order / math.factorial(order), rel_tol=1e-9)
        # dense-grid check that it is the global minimum
        grid = np.linspace(-20, 20, 400001)
        assert T.taylor_weight(grid, order + 1).min() >= w_min - 1e-12
    assert T.truncated_exp_minimum(2)[1] == pytest.approx(0.5, abs=1e-15)
    assert T.truncated_exp_minimum(4)[1] == pytest.approx(0.2703948, abs=1e-7)
    assert T.truncated_exp_minimum(6)[1] == pytest.approx(0.1493248, abs=1e-7)
    # Odd orders have a real root and go negative.
    for order, root in [(1, -1.0), (3, -1.596), (5, -2.181)]:
        t = np.linspace(-10, 0, 1000001)
        w = T.taylor_weight(t, order + 1)
        assert w.min() < 0
        sign_change = t[np.nonzero(np.diff(np.sign(w)))[0][0]]
        assert abs(sign_change - root) < 1e-3


def test_fidelity_sign():
    t = np.linspace(-3, 3, 6001)
    ratio = np.exp(t) / T.taylor_weight(t, 3)
    assert np.all(ratio[t > 1e-9] > 1)
    assert np.all(ratio[t < -1e-9] < 1)
    assert ratio[np.argmin(np.abs(t))] == pytest.approx(1.0, abs=1e-15)


def test_selectivity_law_printed_values():
    g = gold("posfloor_printed.json")["selectivity"]
    w = g["w"]
    based = [T.required_alignment_based(N, w) for N in g["N"]]
    soft = [T.required_alignment_softmax(N, w) for N in g["N"]]
    for x, p, dec in zip(based, g["based"], g["based_decimals"]):
        assert round(x, dec) == p
    for x, p in zip(soft, g["softmax"]):
        assert round(x, g["softmax_decimals"]) == p
    assert round(based[0] / soft[0], g["gap_decimals"][0]) == g["gap_first"]
    assert round(based[-1] / soft[-1], g["gap_decimals"][1]) == g["gap_last"]
    # sqrt(N) tracking: t*/sqrt(N) -> sqrt(w/(1-w)) = 1 from below-ish
    ratios = [b / math.sqrt(N) for b, N in zip(based, g["N"])]
    assert all(abs(r - 1) < 0.15 for r in ratios)
    assert abs(ratios[-1] - 1) < abs(ratios[0] - 1)


def test_selectivity_formula_as_printed_is_the_t0_distractor_law():
    # The printed closed form -1 + sqrt(2(N-1)w/(1-w) - 1) is the law for
    # distractors at t = 0 (weight 1); at N = 64 it gives 10.18, not 6.9.
    for N in (64, 256, 1024, 16384):
        printed = -1 + math.sqrt(2 * (N - 1) * 0.5 / 0.5 - 1)
        assert math.isclose(T.required_alignment_based(N, 0.5, distractor_t=0.0), printed,
                            rel_tol=1e-12)
    assert round(-1 + math.sqrt(2 * 63 - 1), 2) == 10.18


def _selectivity_case(N, distractor_t, d=16, dv=16):
    """Last query e1; N-1 distractor keys at alignment distractor_t (one is
    the query's own); the target key at position 0 carries v = e1."""
    t_star = T.required_alignment_based(N, 0.5, distractor_t=distractor_t)
    q = np.zeros((N, d))
    q[:, 0] = 1.0
    k = np.zeros((N, d))
    k[:, 0] = distractor_t
    k[0, 0] = t_star
    v = np.zeros((N, dv))
    v[0, 0] = 1.0
    return q, k, v


@pytest.mark.parametrize("N", [64, 256, 1024, 16384])
@pytest.mark.parametrize("dt", [-1.0, 0.0])
def test_end_to_end_target_weight(N, dt):
    g = gold("posfloor_printed.json")["selectivity"]
    q, k, v = _selectivity_case(N, dt)
    o = T.direct(q, k, v, 3, 1.0, rows=[N - 1])
    assert abs(o[0, 0] - g["simulated_target_weight"]) < 1e-14
    assert np.all(o[0, 1:] == 0)


# ----------------------------------------------------------------------------
# Special cases of the definition (C-P9)
# ----------------------------------------------------------------------------

def _prefix_mean(v):
    return np.cumsum(v, axis=0) / np.arange(1, len(v) + 1)[:, None]


def test_special_cases():
    rng = np.random.default_rng(3)
    N, d, dv = 40, 5, 3
    q, k, v = (rng.standard_normal((N, d)), rng.standard_normal((N, d)),
               rng.standard_normal((N, dv)))
    assert rel(T.direct(q, k, v, 1, 2.0), _prefix_mean(v)) < 1e-14
    assert rel(T.direct(np.zeros_like(q), k, v, 5, 2.0), _prefix_mean(v)) < 1e-14
    c = np.full((N, dv), 2.5)
    assert np.max(np.abs(T.direct(q, k, c, 3, 2.0) - 2.5)) < 1e-14
    assert rel(T.direct(q[:1], k[:1], v[:1], 3, 2.0), v[:1]) < 1e-15
    kk = np.repeat(k[:1], N, axis=0)
    assert rel(T.direct(q, kk, v, 3, 2.0), _prefix_mean(v)) < 1e-13


# ----------------------------------------------------------------------------
# Reorderings (C-P10): recurrent == direct, direct == exact rationals, additivity
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,dv,n,a", [(4, 3, 3, 2.0), (5, 2, 5, 1.5), (16, 8, 3, 4.0), (3, 4, 1, 1.0)])
def test_recurrent_equals_direct(d, dv, n, a):
    rng = np.random.default_rng(d + dv + n)
    N = 64
    q, k, v = (rng.standard_normal((N, d)), rng.standard_normal((N, d)),
               rng.standard_normal((N, dv)))
    o_rec, S, z = T.recurrent(q, k, v, n, a)
    assert rel(o_rec, T.direct(q, k, v, n, a)) < 1e-12
    S2, z2 = T.state(k, v, n)
    assert rel(S, S2) < 1e-12 and rel(z, z2) < 1e-12


def test_direct_equals_exact_fraction():
    rng = np.random.default_rng(12)
    N, d, dv = 6, 3, 2
    q = rng.integers(-3, 4, (N, d))
    k = rng.integers(-3, 4, (N, d))
    v = rng.integers(-5, 6, (N, dv))
    for n, a in [(3, 1), (5, 2), (1, 3)]:
        ex = T.exact_fraction(q.tolist(), k.tolist(), v.tolist(), n, a)
        ex = np.array([[float(x) for x in row] for row in ex])
        assert rel(T.direct(q, k, v, n, float(a)), ex) < 1e-14


def test_brute_force_double_loop():
    # Pure-Python double loop on a tiny case (no blocking, no masking tricks).
    rng = np.random.default_rng(13)
    N, d, dv, n, a = 9, 4, 3, 3, 2.0
    q, k, v = (rng.standard_normal((N, d)), rng.standard_normal((N, d)),
               rng.standard_normal((N, dv)))
    ref = np.zeros((N, dv))
    for t in range(N):
        num, den = np.zeros(dv), 0.0
        for s in range(t + 1):
            x = float(q[t] @ k[s]) / a
            w = 1.0 + x + x * x / 2.0
            num += w * v[s]
            den += w
        ref[t] = num / den
    assert rel(T.direct(q, k, v, n, a, block=4), ref) < 1e-14


def test_state_additivity_and_continuation():
    rng = np.random.default_rng(14)
    d, dv, n, a = 16, 8, 3, 4.0
    N1, N2 = 50, 30
    q, k, v = (rng.standard_normal((N1 + N2, d)), rng.standard_normal((N1 + N2, d)),
               rng.standard_normal((N1 + N2, dv)))
    S1, z1 = T.state(k[:N1], v[:N1], n)
    S12, z12 = T.state(k[N1:], v[N1:], n, S1, z1)
    Sall, zall = T.state(k, v, n)
    assert rel(S12, Sall) < 1e-13 and rel(z12, zall) < 1e-13
    cont = T.direct(q[N1:], k[N1:], v[N1:], n, a, S0=S1, z0=z1)
    full = T.direct(q, k, v, n, a)[N1:]
    assert rel(cont, full) < 1e-12
    # Segment sums in any grouping give the same total.
    parts = [T.state(k[i:i + 10], v[i:i + 10], n) for i in range(0, N1 + N2, 10)]
    assert rel(sum(p[0] for p in parts), Sall) < 1e-13


def test_decode_step_matches_direct():
    rng = np.random.default_rng(15)
    d, dv, n, a, N = 16, 8, 3, 4.0, 100
    q, k, v = (rng.standard_normal((N, d)), rng.standard_normal((N, d)),
               rng.standard_normal((N, dv)))
    S, z = T.state(k[:N - 3], v[:N - 3], n)
    outs = []
    for t in range(N - 3, N):
        o, S, z = T.decode_step(q[t], k[t], v[t], S, z, n, a)
        outs.append(o)
    ref = T.direct(q, k, v, n, a, rows=[N - 3, N - 2, N - 1])
    assert rel(np.array(outs), ref) < 1e-12


def test_direct_batched_and_rows():
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((2, 3, 20, 4)), rng.standard_normal((2, 3, 20, 4)),
               rng.standard_normal((2, 3, 20, 5)))
    full = T.direct(q, k, v, 3, 2.0)
    assert full.shape == (2, 3, 20, 5)
    assert rel(full[1, 2], T.direct(q[1, 2], k[1, 2], v[1, 2], 3, 2.0)) == 0
    part = T.direct(q, k, v, 3, 2.0, rows=[0, 7, 19])
    assert rel(part, full[:, :, [0, 7, 19]]) < 1e-15


# ----------------------------------------------------------------------------
# Accuracy against softmax (C-P11): the trend only; 6.5e-4 stays unpinned
# ----------------------------------------------------------------------------

def test_softmax_oracle_pins():
    # The softmax reference pinned without its own formula: (1) the Taylor
    # series converges to exp, so direct() with 30 terms equals it when
    # |q.k/a| <= 1/2 (remainder below 1e-40); (2) equal keys give equal
    # weights, i.e. the prefix mean of v; (3) one token returns its value.
    rng = np.random.default_rng(23)
    N, d, dv, a = 96, 16, 8, 2.0
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, dv))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    ref = T.softmax_causal(q, k, v, a, block=40)
    assert rel(ref, T.direct(q, k, v, 30, a)) < 1e-13
    keq = np.repeat(k[:1], N, axis=0)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
    assert rel(T.softmax_causal(q, keq, v, a), prefix_mean) < 1e-14
    assert rel(T.softmax_causal(q[:1], k[:1], v[:1], a), v[:1]) < 1e-15


def test_error_vs_softmax_decreases_with_order():
    rng = np.random.default_rng(17)
    N, d, dv, a = 256, 16, 64, 2.0  # EA defaults, unit-sphere q and k
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, dv))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    ref = T.softmax_causal(q, k, v, a)
    errs = [np.max(np.abs(T.direct(q, k, v, n, a) - ref)) for n in (1, 2, 3, 4, 5)]
    assert all(e1 > e2 for e1, e2 in zip(errs, errs[1:]))
    assert errs[2] < 1e-2  # order 2 already close, consistent in size with EA's 6.5e-4


# ----------------------------------------------------------------------------
# Decayed state (LA, superposed-memory paragraph: a decay multiplying S_{t-1})
# ----------------------------------------------------------------------------

def test_decay_geometric_closed_form():
    # n = 1 (every weight 1) and scalar values v_s = r^s: the decayed average
    # is a ratio of two geometric sums,
    #   o_t = [(r^(t+1) - g^(t+1)) / (r - g)] * [(1 - g) / (1 - g^(t+1))].
    N, g, r = 40, 0.9, 1.03
    rng = np.random.default_rng(5)
    q = rng.standard_normal((N, 4))
    k = rng.standard_normal((N, 4))
    v = (r ** np.arange(N, dtype=np.float64))[:, None]
    t = np.arange(N, dtype=np.float64)
    want = (r ** (t + 1) - g ** (t + 1)) / (r - g) * (1 - g) / (1 - g ** (t + 1))
    assert rel(T.direct(q, k, v, 1, 1.0, gamma=g)[:, 0], want) < 1e-14
    assert rel(T.recurrent(q, k, v, 1, 1.0, gamma=g)[0][:, 0], want) < 1e-13


def test_decay_recurrent_equals_direct_and_limits():
    rng = np.random.default_rng(6)
    N, d, dv, a = 48, 4, 3, 2.0
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, dv))
    for n in (1, 3, 5):
        for g in (0.5, 0.97):
            o_dir = T.direct(q, k, v, n, a, gamma=g)
            o_rec, S, z = T.recurrent(q, k, v, n, a, gamma=g)
            assert rel(o_rec, o_dir) < 1e-12
            S2, z2 = T.state(k, v, n, gamma=g)
            assert rel(S, S2) < 1e-12 and rel(z, z2) < 1e-12
    # gamma = 1 is the plain method; a vanishing gamma keeps only the
    # current token, o_t = v_t
    assert rel(T.direct(q, k, v, 3, a, gamma=1.0), T.direct(q, k, v, 3, a)) == 0
    assert rel(T.direct(q, k, v, 3, a, gamma=1e-30), v) < 1e-15


def test_decay_continuation_through_state():
    # the state after the first part, decayed, carries it exactly: direct on
    # the second part from S0 = state(first part) equals the whole sequence
    rng = np.random.default_rng(7)
    N1, N2, d, dv, a, g = 30, 25, 4, 3, 2.0, 0.93
    q = rng.standard_normal((N1 + N2, d))
    k = rng.standard_normal((N1 + N2, d))
    v = rng.standard_normal((N1 + N2, dv))
    S0, z0 = T.state(k[:N1], v[:N1], 3, gamma=g)
    part = T.direct(q[N1:], k[N1:], v[N1:], 3, a, S0, z0, gamma=g)
    whole = T.direct(q, k, v, 3, a, gamma=g)[N1:]
    assert rel(part, whole) < 1e-13
    o, S, z = T.decode_step(q[N1], k[N1], v[N1], S0, z0, 3, a, gamma=g)
    assert rel(o, whole[0]) < 1e-13


# ----------------------------------------------------------------------------
# Query/key preprocessing (EA: unit-sphere rows are mandatory; temperatures)
# ----------------------------------------------------------------------------

def test_preprocess_pins():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 10, 16))  # [H, N, d]
    x[1, 4] = 0.0                          # a zero row stays zero
    hs = np.array([0.5, 2.0, 3.0])
    y = T.preprocess(x, True, 2.0, hs)
    norms = np.linalg.norm(y, axis=-1)
    want = 2.0 * hs[:, None] * np.ones((3, 10))
    want[1, 4] = 0.0
    assert np.max(np.abs(norms - want)) < 1e-14
    # direction kept, positive rescaling of the input removed
    cos = np.sum(y * x, axis=-1) / np.maximum(norms * np.linalg.norm(x, axis=-1), 1e-300)
    assert np.max(np.abs(cos[norms > 0] - 1)) < 1e-14
    assert rel(T.preprocess(7.5 * x, True, 2.0, hs), y) < 1e-15
    # without normalisation it is a plain rescaling
    assert rel(T.preprocess(x, False, 3.0), 3.0 * x) == 0
