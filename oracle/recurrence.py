"""E -- the eager recurrence, one decode step exactly as the definition states.

[DL] Eq. 3 and the text around it define the common decode step

    S_t = D(lambda_t) S_{t-1} + a_t b_t^T,        o_t = S_t^T q_t,

with D(x) = diag(exp x), lambda_t in R^{d_k} the per-step log-decay (one value
shared by all coordinates for scalar/head-wise decay, a key-wise vector for
diagonal decay), a_t in R^{d_k}, b_t in R^{d_v}, and any query feature map
already folded into q_t.  Linear attention (Eq. 1) is lambda = 0.

Delta-rule operators (DeltaNet, GDN, KDA) build the value-side factor from the
previous state.  The reading used here (the GDN form alpha(I - beta k k^T) S +
beta k v^T, extended to per-key decay as "the delta rule applied to the decayed
state", which is what [DL]'s KDA paragraph describes as keeping GDN's corrected
update while making the decay per key):

    P   = D(lambda_t) S_{t-1}
    a_t = k_t,   b_t = beta_t (v_t - P^T k_t)
    S_t = P + a_t b_t^T

The output reads the post-update state S_t (so it includes the current token).
All arithmetic is float64.  Grouped value heads ([FPGA] system architecture):
v-head h uses q/k head h // (H_v // H_k).
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def expand_heads(x: np.ndarray, H_v: int) -> np.ndarray:
    """[N, H_k, d] -> [N, H_v, d]: v-head h reads q/k head h // (H_v // H_k)."""
    H_k = x.shape[1]
    if H_v % H_k:
        raise ValueError("H_v must be a multiple of H_k")
    return np.repeat(np.asarray(x, dtype=np.float64), H_v // H_k, axis=1)


def decay_factors(lam: Optional[np.ndarray], N: int, H_v: int, d_k: int, decay: str) -> np.ndarray:
    """exp(lambda) as a [N, H_v, d_k] array of row scales (D(lambda)'s diagonal)."""
    if decay == "none":
        return np.ones((N, H_v, d_k))
    lam = np.asarray(lam, dtype=np.float64)
    if decay == "scalar":
        return np.repeat(np.exp(lam)[..., None], d_k, axis=-1)
    if decay == "per_key":
        return np.exp(lam)
    raise ValueError(decay)


def eager_step(S: np.ndarray, q: np.ndarray, a_or_k: np.ndarray, b_or_v: np.ndarray,
               lam: Optional[np.ndarray], beta: Optional[np.ndarray],
               decay: str, update: str) -> Tuple[np.ndarray, np.ndarray]:
    """One step of Eq. 3 for N independent (slot, head-group) states.

    S       [N, H_v, d_k, d_v]  previous states (not modified)
    q       [N, H_k, d_k]
    a_or_k  [N, H_k, d_k]       a_t (plain) or k_t (delta, a_t = k_t)
    b_or_v  [N, H_v, d_v]       b_t (plain) or v_t (delta)
    lam     [N, H_v] (scalar) | [N, H_v, d_k] (per_key) | None (decay "none")
    beta    [N, H_v] for delta, else None
    returns (S_t, o_t) with o_t [N, H_v, d_v]
    """
    S = np.asarray(S, dtype=np.float64)
    N, H_v, d_k, d_v = S.shape
    qv = expand_heads(q, H_v)
    av = expand_heads(a_or_k, H_v)
    g = decay_factors(lam, N, H_v, d_k, decay)
    P = g[..., :, None] * S                                   # D(lambda) S: scales rows
    if update == "delta":
        PTk = np.matmul(np.swapaxes(P, -1, -2), av[..., None])[..., 0]
        b = np.asarray(beta, dtype=np.float64)[..., None] * (np.asarray(b_or_v, dtype=np.float64) - PTk)
    elif update == "plain":
        b = np.asarray(b_or_v, dtype=np.float64)
    else:
        raise ValueError(update)
    S_new = P + av[..., :, None] * b[..., None, :]           # + a b^T
    o = np.matmul(np.swapaxes(S_new, -1, -2), qv[..., None])[..., 0]   # S_t^T q
    return S_new, o
