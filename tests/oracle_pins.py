"""Pins for the oracle: each returns an error that must be ~0 for a correct oracle.

Every pin takes the step function (or pool class) under test as an argument, so
the mutation tests can hand it a copy of the oracle with a planted mistake and
check that some pin catches it.  Inputs are small, seeded and local to the pin.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from oracle import closed_forms as cf
from oracle import schedule
from oracle.deferred import DeferredPool
from oracle.recurrence import eager_step


def _rel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _run_single_head(step, S0, q, a, b, lam, beta, decay, update):
    """Drive a step function over T tokens for one head; returns (states, outputs)."""
    T = q.shape[0]
    S = S0[None, None]
    states, outs = [], []
    for t in range(T):
        lt = None
        if decay == "scalar":
            lt = np.array([[lam[t]]])
        elif decay == "per_key":
            lt = lam[t][None, None]
        bt = None if beta is None else np.array([[beta[t]]])
        S, o = step(S, q[t][None, None], a[t][None, None], b[t][None, None], lt, bt, decay, update)
        states.append(S[0, 0].copy())
        outs.append(o[0, 0].copy())
    return states, outs


# ------------------------------------------------------------------- E pins
def pin_plain_closed_form(step=eager_step, seed=0, d_k=6, d_v=6, T=12) -> float:
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((d_k, d_v))
    q, a = rng.standard_normal((T, d_k)), rng.standard_normal((T, d_k))
    b = rng.standard_normal((T, d_v))
    states, outs = _run_single_head(step, S0, q, a, b, None, None, "none", "plain")
    S_ref, o_ref = cf.plain_closed_form(a, b, q, S0)
    return max(_rel(states[-1], S_ref), _rel(np.array(outs), o_ref))


def pin_decayed_closed_form(step=eager_step, decay="per_key", seed=1, d=6, T=10) -> float:
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((d, d))
    q, a, b = (rng.standard_normal((T, d)) for _ in range(3))
    if decay == "per_key":
        lam = -rng.uniform(0.05, 1.0, size=(T, d))
        lam_full = lam
    else:
        lam = -rng.uniform(0.05, 1.0, size=T)
        lam_full = np.repeat(lam[:, None], d, axis=1)
    states, outs = _run_single_head(step, S0, q, a, b, lam, None, decay, "plain")
    S_ref, o_ref = cf.decayed_closed_form(S0, lam_full, a, b, q)
    return max(_rel(states[-1], S_ref), _rel(np.array(outs), o_ref))


def pin_delta_product_form(step=eager_step, decay="per_key", seed=2, d=6, T=8) -> float:
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((d, d))
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    beta = rng.uniform(0.1, 0.9, size=T)
    if decay == "per_key":
        lam = -rng.uniform(0.05, 1.0, size=(T, d))
        lam_full = lam
    else:
        lam = -rng.uniform(0.05, 1.0, size=T)
        lam_full = np.repeat(lam[:, None], d, axis=1)
    states, outs = _run_single_head(step, S0, q, k, v, lam, beta, decay, "delta")
    err = 0.0
    for t in range(T):
        S_ref = cf.delta_product_form(S0, lam_full[: t + 1], k[: t + 1], v[: t + 1], beta[: t + 1])
        err = max(err, _rel(states[t], S_ref), _rel(outs[t], S_ref.T @ q[t]))
    return err


def pin_delta_identity(step=eager_step, decay="scalar", seed=3, d=7) -> float:
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((d, d))
    k, v, q = (rng.standard_normal(d) for _ in range(3))
    beta = 0.37
    lam = -0.3 if decay == "scalar" else -rng.uniform(0.05, 1.0, size=d)
    lam_full = np.full(d, lam) if decay == "scalar" else lam
    states, outs = _run_single_head(step, S, q[None], k[None], v[None],
                                    np.atleast_1d(lam) if decay == "scalar" else lam[None],
                                    np.array([beta]), decay, "delta")
    ref = cf.delta_identity(S, lam_full, k, v, beta)
    return max(_rel(states[0], ref), _rel(outs[0], ref.T @ q))


def pin_beta_one_recall(step=eager_step, decay="scalar", seed=4, d=8, T=6) -> float:
    """beta = 1 and ||k|| = 1: the new state maps k_t exactly to v_t (S_t^T k_t = v_t)."""
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((d, d))
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    lam = -rng.uniform(0.05, 1.0, size=(T, d) if decay == "per_key" else T)
    states, _ = _run_single_head(step, S0, q, k, v, lam, np.ones(T), decay, "delta")
    return max(_rel(states[t].T @ k[t], v[t]) for t in range(T))


def pin_beta_zero_decay_only(step=eager_step, decay="per_key", seed=5, d=6, T=5) -> float:
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((d, d))
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    lam = -rng.uniform(0.05, 1.0, size=(T, d) if decay == "per_key" else T)
    states, outs = _run_single_head(step, S0, q, k, v, lam, np.zeros(T), decay, "delta")
    S = S0
    err = 0.0
    for t in range(T):
        g = np.exp(lam[t]) if decay == "per_key" else np.full(d, math.exp(lam[t]))
        S = g[:, None] * S
        err = max(err, _rel(states[t], S), _rel(outs[t], S.T @ q[t]))
    return err


def _frac_vec(rng, n, denom=8, lo=-8, hi=8):
    return [Fraction(int(x), denom) for x in rng.integers(lo, hi + 1, size=n)]


def pin_exact_rational(step=eager_step, decay="per_key", update="delta", seed=6, d=4, T=12) -> float:
    """fp64 oracle vs exact rational arithmetic (alpha rational, lam = log alpha)."""
    rng = np.random.default_rng(seed)
    S0 = [_frac_vec(rng, d, 16) for _ in range(d)]
    if decay == "none":
        alpha = [[Fraction(1)] * d for _ in range(T)]
    elif decay == "scalar":
        alpha = []
        for _ in range(T):
            x = Fraction(int(rng.integers(9, 16)), 16)
            alpha.append([x] * d)
    else:
        alpha = [[Fraction(int(x), 16) for x in rng.integers(9, 16, size=d)] for _ in range(T)]
    q = [_frac_vec(rng, d) for _ in range(T)]
    k = [_frac_vec(rng, d) for _ in range(T)]
    v = [_frac_vec(rng, d) for _ in range(T)]
    beta = [Fraction(int(x), 8) for x in rng.integers(1, 8, size=T)] if update == "delta" else None
    ex_states, ex_outs = cf.exact_rational_run(S0, alpha, q, k, v, beta, update)

    f = lambda m: np.array([[float(x) for x in row] for row in m])
    lam = None
    if decay == "scalar":
        lam = np.array([math.log(alpha[t][0]) for t in range(T)])
    elif decay == "per_key":
        lam = np.array([[math.log(x) for x in alpha[t]] for t in range(T)])
    states, outs = _run_single_head(step, f(S0), f(q), f(k), f(v), lam,
                                    None if beta is None else np.array([float(b) for b in beta]),
                                    decay, update)
    err = 0.0
    for t in range(T):
        err = max(err, _rel(states[t], f(ex_states[t])),
                  _rel(outs[t], np.array([float(x) for x in ex_outs[t]])))
    return err


def pin_grouped_heads(step=eager_step, seed=7, H_v=4, H_k=2, d=5) -> float:
    """Grouped value heads equal the same step with q/k copied to every v-head by hand."""
    rng = np.random.default_rng(seed)
    N = 3
    S = rng.standard_normal((N, H_v, d, d))
    q, k = rng.standard_normal((N, H_k, d)), rng.standard_normal((N, H_k, d))
    v = rng.standard_normal((N, H_v, d))
    lam = -rng.uniform(0.05, 1.0, size=(N, H_v, d))
    beta = rng.uniform(0.1, 0.9, size=(N, H_v))
    S1, o1 = step(S, q, k, v, lam, beta, "per_key", "delta")
    qf = np.zeros((N, H_v, d))
    kf = np.zeros((N, H_v, d))
    group = H_v // H_k
    for h in range(H_v):
        for g in range(H_k):
            if g * group <= h < (g + 1) * group:
                qf[:, h], kf[:, h] = q[:, g], k[:, g]
    err = 0.0
    for h in range(H_v):
        S2, o2 = step(S[:, h:h + 1], qf[:, h:h + 1], kf[:, h:h + 1], v[:, h:h + 1],
                      lam[:, h:h + 1], beta[:, h:h + 1], "per_key", "delta")
        err = max(err, _rel(S1[:, h], S2[:, 0]), _rel(o1[:, h], o2[:, 0]))
    return err


E_PINS = {
    "plain_closed_form": lambda s: pin_plain_closed_form(s),
    "plain_closed_form_rect": lambda s: pin_plain_closed_form(s, d_k=4, d_v=7),
    "decayed_closed_form_per_key": lambda s: pin_decayed_closed_form(s, "per_key"),
    "decayed_closed_form_scalar": lambda s: pin_decayed_closed_form(s, "scalar"),
    "delta_product_per_key": lambda s: pin_delta_product_form(s, "per_key"),
    "delta_product_scalar": lambda s: pin_delta_product_form(s, "scalar"),
    "delta_identity_scalar": lambda s: pin_delta_identity(s, "scalar"),
    "delta_identity_per_key": lambda s: pin_delta_identity(s, "per_key"),
    "beta_one_scalar": lambda s: pin_beta_one_recall(s, "scalar"),
    "beta_one_per_key": lambda s: pin_beta_one_recall(s, "per_key"),
    "beta_zero": lambda s: pin_beta_zero_decay_only(s),
    "exact_plain_none": lambda s: pin_exact_rational(s, "none", "plain"),
    "exact_plain_per_key": lambda s: pin_exact_rational(s, "per_key", "plain"),
    "exact_delta_scalar": lambda s: pin_exact_rational(s, "scalar", "delta"),
    "exact_delta_per_key": lambda s: pin_exact_rational(s, "per_key", "delta"),
    "grouped_heads": lambda s: pin_grouped_heads(s),
}


# ------------------------------------------------------------------- F pins
def pin_deferred_equals_eager(pool_cls=DeferredPool, step=eager_step, decay="per_key",
                              update="delta", L=4, seed=8, P=5, H_v=4, H_k=2, d=6, T=23) -> float:
    """Logical state of base + log == eager state at every step; outputs equal;
    the base right after a merge equals the eager state."""
    rng = np.random.default_rng(seed)
    F = pool_cls(P, H_v, H_k, d, d, L, decay, update)
    init = rng.standard_normal((P, H_v, d, d)) * 0.3
    F.assign(range(P), init)
    E = init.copy()
    err = 0.0
    for t in range(T):
        B = int(rng.integers(1, P + 1))
        slots = rng.choice(P, size=B, replace=False)
        q, k = rng.standard_normal((B, H_k, d)), rng.standard_normal((B, H_k, d))
        v = rng.standard_normal((B, H_v, d))
        lam = None
        if decay == "scalar":
            lam = -rng.uniform(0.01, 0.5, size=(B, H_v))
        elif decay == "per_key":
            lam = -rng.uniform(0.01, 0.5, size=(B, H_v, d))
        beta = rng.uniform(0.1, 0.9, size=(B, H_v)) if update == "delta" else None
        nbefore = F.n[slots].copy()
        o_f, _ = F.step(slots, q, k, v, lam, beta)
        S_e, o_e = step(E[slots], q, k, v, lam, beta, decay, update)
        E[slots] = S_e
        err = max(err, _rel(o_f, o_e))
        for j, s in enumerate(slots):
            err = max(err, _rel(F.logical_state(int(s)), E[s]))
            if nbefore[j] == F.C:          # this step merged: the base is the state
                err = max(err, _rel(F.base[s], E[s]))
    F.flush_all()
    err = max(err, _rel(F.base, E))
    return err


def pin_schedule_closed_form(pool_cls=DeferredPool, L=5, seed=9, P=7, T=60) -> int:
    """Number of (step, slot) decisions where the deferred pool's bookkeeping
    differs from the closed form, with fresh assignments and explicit merges."""
    rng = np.random.default_rng(seed)
    d, H = 2, 1
    F = pool_cls(P, H, H, d, d, L, "scalar", "plain")
    Cn = schedule.Counters(P, L)
    bad = 0
    for t in range(T):
        if t % 7 == 3:
            rs = rng.choice(P, size=2, replace=False)
            F.assign(rs, np.zeros((2, H, d, d)))
            Cn.reset(rs)
        if t % 11 == 5:
            ms = rng.choice(P, size=2, replace=False)
            F.merge(ms)
            Cn.merge(ms)
        B = int(rng.integers(1, P + 1))
        slots = rng.choice(P, size=B, replace=False)
        x = rng.standard_normal((B, H, d))
        _, got = F.step(slots, x, x, x, -np.ones((B, H)) * 0.1, None)
        want = Cn.decode(slots)
        bad += sum(int(g != w) for g, w in zip(got, want))
        bad += int(np.sum(F.n != Cn.n))
    return bad
