"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Each mutation swaps one function of ``oracle.taylor_oracle`` for a subtly
wrong copy; the pin tests of test_oracle_pins.py are then run against the
mutated module and at least one of them must fail.
"""
import inspect
import itertools
import math

import numpy as np
import pytest

from oracle import taylor_oracle as T
import tests.test_oracle_pins as P


def _weight_no_factorial(t, n_terms):
    total, power = 0 * t, 1 + 0 * t
    for m in range(n_terms):
        total = total + power
        power = power * t
    return total


def _weight_drop_last(t, n_terms):
    total, power = 0 * t, 1 + 0 * t
    for m in range(n_terms - 1):
        total = total + power / math.factorial(m)
        power = power * t
    return total


def _multinomial_one(tup):
    return 1


def _monomials_strict(d, m):
    return list(itertools.combinations(range(d), m))


_orig_direct = T.direct


def _direct_sign_flip(q, k, v, n_terms, a, *args, **kw):
    return _orig_direct(q, -np.asarray(k, dtype=np.float64), v, n_terms, a, *args, **kw)


def _direct_shifted_mask(q, k, v, n_terms, a, S0=None, z0=None, rows=None, block=256):
    # drops the diagonal term s == t (exclusive mask), keeping row 0 defined
    q = np.asarray(q, dtype=np.float64)
    if q.ndim > 2:
        return _orig_direct(q, k, v, n_terms, a, S0, z0, rows, block)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N = q.shape[0]
    sel = np.arange(N) if rows is None else np.asarray(rows)
    W = T.taylor_weight(q[sel] @ k.T / a, n_terms)
    mask = (np.arange(N)[None, :] < sel[:, None]) | ((sel[:, None] == 0) & (np.arange(N)[None, :] == 0))
    W = np.where(mask, W, 0.0)
    out = (W @ v) / W.sum(1)[:, None]
    if S0 is not None:
        return _orig_direct(q, k, v, n_terms, a, S0, z0, rows, block)
    return out


def _recurrent_read_first(q, k, v, n_terms, a, S0=None, z0=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    F = T.n_features(d, n_terms)
    S = np.zeros((F, v.shape[1]))
    z = np.zeros(F)
    alpha = T.alpha_vector(d, n_terms, a)
    out = np.empty((N, v.shape[1]))
    for t in range(N):
        fq = T.phi(q[t:t + 1], n_terms)[0] * alpha
        fk = T.phi(k[t:t + 1], n_terms)[0]
        if t == 0:
            S, z = S + np.outer(fk, v[t]), z + fk
            out[t] = (fq @ S) / (fq @ z)
            continue
        out[t] = (fq @ S) / (fq @ z)
        S, z = S + np.outer(fk, v[t]), z + fk
    return out, S, z


def _alpha_no_factorial(d, n_terms, a):
    out = []
    for m in range(n_terms):
        out += [1.0 / a ** m] * math.comb(d + m - 1, m)
    return np.array(out)


def _direct_decay_bug(kind):
    """Decayed direct form with one planted mistake: 'den' leaves the
    denominator undecayed, 's0' carries S0 with gamma^t instead of gamma^(t+1)."""
    def f(q, k, v, n_terms, a, S0=None, z0=None, rows=None, block=256, gamma=1.0):
        q = np.asarray(q, dtype=np.float64)
        if q.ndim > 2 or gamma == 1.0:
            return _orig_direct(q, k, v, n_terms, a, S0, z0, rows, block, gamma)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        N = q.shape[0]
        r = np.arange(N) if rows is None else np.asarray(rows)
        W = T.taylor_weight(q[r] @ k.T / a, n_terms)
        lag = r[:, None] - np.arange(N)[None, :]
        W = np.where(lag >= 0, W, 0.0)
        Wd = W * np.power(gamma, np.maximum(lag, 0).astype(np.float64))
        num = Wd @ v
        den = (W if kind == "den" else Wd).sum(1)
        if S0 is not None:
            fq = T.phi(q[r], n_terms) * T.alpha_vector(q.shape[1], n_terms, a)
            carry = np.power(gamma, r + (0.0 if kind == "s0" else 1.0))
            num = num + carry[:, None] * (fq @ np.asarray(S0))
            den = den + carry * (fq @ np.asarray(z0))
        return num / den[:, None]
    return f


_orig_recurrent = T.recurrent


def _recurrent_decay_after_write(q, k, v, n_terms, a, S0=None, z0=None, gamma=1.0):
    if gamma == 1.0:
        return _orig_recurrent(q, k, v, n_terms, a, S0, z0)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    F = T.n_features(d, n_terms)
    S = np.zeros((F, v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64)
    z = np.zeros(F) if z0 is None else np.array(z0, dtype=np.float64)
    alpha = T.alpha_vector(d, n_terms, a)
    out = np.empty((N, v.shape[1]))
    for t in range(N):
        fk = T.phi(k[t:t + 1], n_terms)[0]
        S = gamma * (S + np.outer(fk, v[t]))
        z = gamma * (z + fk)
        fq = T.phi(q[t:t + 1], n_terms)[0] * alpha
        out[t] = (fq @ S) / (fq @ z)
    return out, S, z


def _alignment_printed(N, w, distractor_t=-1.0):
    return -1 + math.sqrt(2 * (N - 1) * w / (1 - w) - 1)


MUTATIONS = {
    "weight_without_factorials": ("taylor_weight", _weight_no_factorial),
    "weight_drops_last_term": ("taylor_weight", _weight_drop_last),
    "phi_without_multinomial_weights": ("multinomial", _multinomial_one),
    "basis_without_repeated_indices": ("monomials", _monomials_strict),
    "direct_wrong_sign": ("direct", _direct_sign_flip),
    "direct_exclusive_mask": ("direct", _direct_shifted_mask),
    "recurrent_reads_before_update": ("recurrent", _recurrent_read_first),
    "alpha_without_factorials": ("alpha_vector", _alpha_no_factorial),
    "alignment_printed_formula": ("required_alignment_based", _alignment_printed),
    "decay_leaves_denominator": ("direct", _direct_decay_bug("den")),
    "decay_initial_state_one_step_short": ("direct", _direct_decay_bug("s0")),
    "decay_after_the_write": ("recurrent", _recurrent_decay_after_write),
}


def _pin_tests():
    tests = []
    for name, fn in inspect.getmembers(P, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            tests.append((name, fn, {}))
            continue
        # expand (possibly stacked) parametrizations
        grids = []
        for m in params:
            names = [s.strip() for s in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(names, v)) for v in vals])
        for combo in itertools.product(*grids):
            kw = {}
            for c in combo:
                kw.update(c)
            tests.append((name, fn, kw))
    return tests


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(mutation, monkeypatch):
    attr, bad = MUTATIONS[mutation]
    monkeypatch.setattr(T, attr, bad)
    caught = []
    for name, fn, kw in _pin_tests():
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(name)
    assert caught, f"no pin caught mutation {mutation}"


def test_unmutated_oracle_passes_every_pin():
    for name, fn, kw in _pin_tests():
        fn(**kw)
