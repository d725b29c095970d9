"""Closed forms and exact arithmetic that pin the recurrence from outside.

Single-head helpers (no batch / head axes) written as sums and products over the
whole token history rather than as a step-by-step recurrence, so that a mistake
in the recurrence code (a dropped term, a wrong sign, a transposed operand, the
output read from the wrong state) shows up as a disagreement.

* plain_closed_form    [DL] Eq. 1 unrolled: S_T = S_0 + sum_t a_t b_t^T,
                       o_t = S_t^T q_t = S_0^T q_t + sum_{s<=t} (a_s . q_t) b_s
* decayed_closed_form  Eq. 3 with a raw value unrolled:
                       S_t = D(sum_{s<=t} lam_s) S_0 + sum_{u<=t} D(sum_{u<s<=t} lam_s) a_u b_u^T
                       (the same algebra as [DL]'s logical-state equation)
* delta_product_form   delta rule as a product of transition matrices:
                       S_T = (A_T ... A_1) S_0 + sum_t (A_T ... A_{t+1}) beta_t k_t v_t^T,
                       A_t = (I - beta_t k_t k_t^T) D(lam_t)
* delta_identity       one delta step written as alpha (I - beta k k^T) S + beta k v^T
                       (GDN's form), or (I - beta k k^T) D S + beta k v^T (per key)
* exact_rational_run   the decode step in exact rational arithmetic (Python
                       ``fractions``) with a rational decay alpha = exp(lambda),
                       index by index over plain nested lists, for d = 4.
"""

from __future__ import annotations

from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np


def plain_closed_form(a_seq: np.ndarray, b_seq: np.ndarray, q_seq: np.ndarray,
                      S0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """No decay, b given.  a_seq [T,d_k], b_seq [T,d_v], q_seq [T,d_k] -> (S_T, o [T,d_v])."""
    a_seq, b_seq, q_seq = (np.asarray(x, dtype=np.float64) for x in (a_seq, b_seq, q_seq))
    T, d_k = a_seq.shape
    d_v = b_seq.shape[1]
    S0 = np.zeros((d_k, d_v)) if S0 is None else np.asarray(S0, dtype=np.float64)
    o = np.zeros((T, d_v))
    for t in range(T):
        o[t] = S0.T @ q_seq[t]
        for s in range(t + 1):
            o[t] += float(a_seq[s] @ q_seq[t]) * b_seq[s]
    S_T = S0 + sum(np.outer(a_seq[t], b_seq[t]) for t in range(T))
    return S_T, o


def decayed_closed_form(S0: np.ndarray, lam_seq: np.ndarray, a_seq: np.ndarray,
                        b_seq: np.ndarray, q_seq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-key log-decay lam_seq [T,d_k] (broadcast a scalar decay before calling)."""
    S0, lam_seq, a_seq, b_seq, q_seq = (np.asarray(x, dtype=np.float64)
                                        for x in (S0, lam_seq, a_seq, b_seq, q_seq))
    T = lam_seq.shape[0]
    o = np.zeros((T, b_seq.shape[1]))
    S_t = S0
    for t in range(T):
        total = lam_seq[: t + 1].sum(axis=0)                     # sum_{s<=t} lam_s
        S_t = np.exp(total)[:, None] * S0
        for u in range(t + 1):
            after = lam_seq[u + 1: t + 1].sum(axis=0)            # sum_{u<s<=t} lam_s
            S_t = S_t + np.exp(after)[:, None] * np.outer(a_seq[u], b_seq[u])
        o[t] = S_t.T @ q_seq[t]
    return S_t, o


def delta_product_form(S0: np.ndarray, lam_seq: np.ndarray, k_seq: np.ndarray,
                       v_seq: np.ndarray, beta_seq: np.ndarray) -> np.ndarray:
    """S_T of the delta rule via transition matrices A_t = (I - beta k k^T) D(lam_t)."""
    S0, lam_seq, k_seq, v_seq = (np.asarray(x, dtype=np.float64) for x in (S0, lam_seq, k_seq, v_seq))
    beta_seq = np.asarray(beta_seq, dtype=np.float64)
    T, d_k = k_seq.shape
    A = [(np.eye(d_k) - beta_seq[t] * np.outer(k_seq[t], k_seq[t])) @ np.diag(np.exp(lam_seq[t]))
         for t in range(T)]

    def prod(lo: int) -> np.ndarray:            # A_{T-1} ... A_lo  (0-based)
        M = np.eye(d_k)
        for t in range(lo, T):
            M = A[t] @ M
        return M

    S_T = prod(0) @ S0
    for t in range(T):
        S_T = S_T + prod(t + 1) @ (beta_seq[t] * np.outer(k_seq[t], v_seq[t]))
    return S_T


def delta_identity(S: np.ndarray, lam: np.ndarray, k: np.ndarray, v: np.ndarray, beta: float) -> np.ndarray:
    """(I - beta k k^T) D(lam) S + beta k v^T; for a scalar decay alpha = e^lam this is
    alpha (I - beta k k^T) S + beta k v^T."""
    S, lam, k, v = (np.asarray(x, dtype=np.float64) for x in (S, lam, k, v))
    d_k = S.shape[0]
    return (np.eye(d_k) - beta * np.outer(k, k)) @ (np.exp(lam)[:, None] * S) + beta * np.outer(k, v)


# ----------------------------------------------------------- exact rationals
def _mat(rows: int, cols: int) -> List[List[Fraction]]:
    return [[Fraction(0) for _ in range(cols)] for _ in range(rows)]


def exact_rational_run(S0: Sequence[Sequence[Fraction]], alpha: Sequence[Sequence[Fraction]],
                       q: Sequence[Sequence[Fraction]], a_or_k: Sequence[Sequence[Fraction]],
                       b_or_v: Sequence[Sequence[Fraction]], beta: Optional[Sequence[Fraction]],
                       update: str):
    """Exact decode of one head.  alpha[t][r] = exp(lam_t[r]) as a rational.

    Every quantity is a Fraction and every sum is written index by index:
        P[r][c]  = alpha[t][r] * S[r][c]
        b[c]     = beta_t * (v[c] - sum_r P[r][c] * k[r])   (delta) | given b[c]
        S[r][c]  = P[r][c] + a[r] * b[c]
        o[c]     = sum_r S[r][c] * q[r]
    Returns (list of states after each step, list of outputs).
    """
    d_k, d_v = len(S0), len(S0[0])
    S = [[Fraction(x) for x in row] for row in S0]
    states, outs = [], []
    for t in range(len(q)):
        P = _mat(d_k, d_v)
        for r in range(d_k):
            for c in range(d_v):
                P[r][c] = alpha[t][r] * S[r][c]
        a = list(a_or_k[t])
        if update == "delta":
            b = []
            for c in range(d_v):
                proj = sum((P[r][c] * a[r] for r in range(d_k)), Fraction(0))
                b.append(beta[t] * (b_or_v[t][c] - proj))
        else:
            b = list(b_or_v[t])
        S = _mat(d_k, d_v)
        for r in range(d_k):
            for c in range(d_v):
                S[r][c] = P[r][c] + a[r] * b[c]
        o = [sum((S[r][c] * q[t][r] for r in range(d_k)), Fraction(0)) for c in range(d_v)]
        states.append([row[:] for row in S])
        outs.append(o)
    return states, outs
