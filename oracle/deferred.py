"""F -- the deferred (base + log) representation, following [DL]'s design section.

Physical state of one slot ([DL], the physical-state list), per head:
  S_bar   dense base                               [d_k, d_v]
  l_bar   cumulative log-decay since the last materialization:
          one value per head (scalar decay) or one per key (per-key decay)
  K_log   deferred key-side factors  a_i           [C, d_k]
  U_log   deferred value-side factors b_i          [C, d_v]
  Lam_log log-decay snapshot per entry (same structure as l_bar)
  n       live-log length, 0 <= n <= C
with M the merge interval and C = M - 1 the live-log capacity.  Here M is the
workload's L.

Logical state ([DL], the logical-state equation and the sentence after it):
  S = D(l_bar) S_bar + sum_{i<n} D(l_bar - Lam_log[i]) K_log[i] U_log[i]^T
the first term is the base decayed by everything since materialization, the
second replays each entry with the decay accumulated after it was inserted.
That sentence fixes the snapshot convention: Lam_log[i] is l_bar right after
the inserting step's own decay was added, so the newest entry replays with
weight exp(0) = 1.

One decode step ([DL] Algorithm 1 / the append-merge cycle, and the
ReplayPrep / AppendDecode / Finalize / Merge description of its GPU section):
  l'      = l_bar + lambda_t
  P^T x   = S_bar^T (e^{l'} * x) + sum_i ((e^{l' - Lam_i} * K_i) . x) U_i
            (P = D(lambda_t) S_{t-1} is never formed; x is q_t or k_t)
  b_t     = beta_t (v_t - P^T k_t)  [delta]   or the given b_t [plain]
  o_t     = P^T q_t + (a_t . q_t) b_t          (= S_t^T q_t)
  append (n < C):  K_n <- a_t, U_n <- b_t, Lam_n <- l', l_bar <- l', n <- n + 1
  merge  (n = C):  S_bar <- D(l') S_bar + sum_i D(l' - Lam_i) K_i U_i^T + a_t b_t^T,
                   l_bar <- 0, n <- 0
so a cycle is C appends then one merge, one dense write per M tokens.

Slot (re)assignment follows [DL]'s allocator paragraph: a fresh slot takes the
given dense state as its base with an empty auxiliary representation.

Float64 throughout; nothing is rounded to a storage dtype.
"""

from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .recurrence import expand_heads


class DeferredPool:
    APPEND, MERGE = 0, 1

    def __init__(self, num_slots: int, H_v: int, H_k: int, d_k: int, d_v: int,
                 L: int, decay: str, update: str):
        if L < 1:
            raise ValueError("merge interval must be >= 1")
        if decay not in ("none", "scalar", "per_key") or update not in ("plain", "delta"):
            raise ValueError((decay, update))
        self.P, self.H_v, self.H_k, self.d_k, self.d_v = num_slots, H_v, H_k, d_k, d_v
        self.M, self.C = L, L - 1
        self.decay, self.update = decay, update
        w = d_k if decay == "per_key" else 1          # one value per head, or per key
        self.base = np.zeros((num_slots, H_v, d_k, d_v))
        self.lbar = np.zeros((num_slots, H_v, w))
        self.K = np.zeros((num_slots, H_v, max(self.C, 1), d_k))
        self.U = np.zeros((num_slots, H_v, max(self.C, 1), d_v))
        self.Lam = np.zeros((num_slots, H_v, max(self.C, 1), w))
        self.n = np.zeros(num_slots, dtype=np.int64)
        self.merges = np.zeros(num_slots, dtype=np.int64)

    # ------------------------------------------------------------ allocator
    def assign(self, slots, states: Optional[np.ndarray] = None) -> None:
        for j, s in enumerate(np.asarray(slots, dtype=np.int64)):
            self.base[s] = 0.0 if states is None else np.asarray(states[j], dtype=np.float64)
            self.lbar[s] = 0.0
            self.n[s] = 0

    # -------------------------------------------------------- logical state
    def logical_state(self, s: int) -> np.ndarray:
        """D(l_bar) S_bar + sum_{i<n} D(l_bar - Lam_i) K_i U_i^T for slot s."""
        n = int(self.n[s])
        S = np.exp(self.lbar[s])[:, :, None] * self.base[s]
        for i in range(n):
            w = np.exp(self.lbar[s] - self.Lam[s, :, i])            # [H_v, 1 or d_k]
            S = S + (w * self.K[s, :, i])[:, :, None] * self.U[s, :, i][:, None, :]
        return S

    def logical_states(self, slots) -> np.ndarray:
        return np.stack([self.logical_state(int(s)) for s in slots])

    # ------------------------------------------------------------- one step
    def _lam_vec(self, lam_e: Optional[np.ndarray]) -> np.ndarray:
        if self.decay == "none":
            return np.zeros((self.H_v, 1))
        lam_e = np.asarray(lam_e, dtype=np.float64)
        return lam_e[:, None] if self.decay == "scalar" else lam_e

    def _replay_transpose(self, s: int, lprime: np.ndarray, x: np.ndarray) -> np.ndarray:
        """P^T x from base + log, P = D(l') S_bar + sum_i D(l' - Lam_i) K_i U_i^T."""
        y = np.einsum("hrc,hr->hc", self.base[s], np.exp(lprime) * x)
        for i in range(int(self.n[s])):
            c = np.sum(np.exp(lprime - self.Lam[s, :, i]) * self.K[s, :, i] * x, axis=-1)  # [H_v]
            y = y + c[:, None] * self.U[s, :, i]
        return y

    def step(self, slots, q, a_or_k, b_or_v, lam=None, beta=None
             ) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Decode one token for each slot in ``slots`` (distinct).

        Returns the outputs o_t [B, H_v, d_v] and, per entry, (phase, index):
        phase MERGE or APPEND, index = the log position written (append) or the
        live length replayed (merge).
        """
        slots = np.asarray(slots, dtype=np.int64)
        if len(set(slots.tolist())) != len(slots):
            raise ValueError("slot ids in one step must be distinct")
        B = len(slots)
        qv = expand_heads(q, self.H_v)
        av = expand_heads(a_or_k, self.H_v)
        bv = np.asarray(b_or_v, dtype=np.float64)
        out = np.zeros((B, self.H_v, self.d_v))
        sched = []
        for e, s in enumerate(slots):
            lprime = self.lbar[s] + self._lam_vec(None if lam is None else lam[e])
            a = av[e]
            if self.update == "delta":
                b = np.asarray(beta[e], dtype=np.float64)[:, None] * (bv[e] - self._replay_transpose(s, lprime, a))
            else:
                b = bv[e]
            out[e] = self._replay_transpose(s, lprime, qv[e]) + np.sum(a * qv[e], axis=-1)[:, None] * b
            n = int(self.n[s])
            if n == self.C:
                S = np.exp(lprime)[:, :, None] * self.base[s]
                for i in range(n):
                    w = np.exp(lprime - self.Lam[s, :, i])
                    S = S + (w * self.K[s, :, i])[:, :, None] * self.U[s, :, i][:, None, :]
                self.base[s] = S + a[:, :, None] * b[:, None, :]
                self.lbar[s] = 0.0
                self.n[s] = 0
                self.merges[s] += 1
                sched.append((self.MERGE, n))
            else:
                self.K[s, :, n] = a
                self.U[s, :, n] = b
                self.Lam[s, :, n] = lprime
                self.lbar[s] = lprime
                self.n[s] = n + 1
                sched.append((self.APPEND, n))
        return out, sched

    # ------------------------------------------------------- explicit merge
    def merge(self, slots) -> None:
        """Materialize the logical state into the base and clear the log.

        A slot with an empty log is left untouched.
        """
        for s in np.asarray(slots, dtype=np.int64):
            if self.n[s] == 0:
                continue
            self.base[s] = self.logical_state(int(s))
            self.lbar[s] = 0.0
            self.n[s] = 0

    def flush_all(self) -> None:
        self.merge(np.nonzero(self.n > 0)[0])
