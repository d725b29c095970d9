"""A slot pool driven by E, tracking only a chosen subset of slots.

Slots are independent ([DL] decode-phase section: one state slot per request
per layer), so the eager recurrence of a sampled subset of a large serving pool
is exact for those slots.  The pool applies, per step, the fresh-state
assignments first and then the decode of every tracked entry, in the order the
workload gives them.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .recurrence import eager_step


class EagerPool:
    def __init__(self, tracked: Sequence[int], H_v: int, d_k: int, d_v: int,
                 decay: str, update: str, init: Optional[np.ndarray] = None):
        self.tracked = [int(s) for s in tracked]
        self.row = {s: i for i, s in enumerate(self.tracked)}
        self.decay, self.update = decay, update
        self.S = np.zeros((len(self.tracked), H_v, d_k, d_v))
        if init is not None:
            self.S[:] = np.asarray(init, dtype=np.float64)

    def assign(self, slots: Sequence[int], states: np.ndarray) -> None:
        for j, s in enumerate(slots):
            r = self.row.get(int(s))
            if r is not None:
                self.S[r] = np.asarray(states[j], dtype=np.float64)

    def entries(self, slot_ids: Sequence[int]) -> np.ndarray:
        """Batch positions whose slot is tracked."""
        return np.array([e for e, s in enumerate(slot_ids) if int(s) in self.row], dtype=np.int64)

    def step(self, slot_ids, q, a_or_k, b_or_v, lam=None, beta=None):
        """Decode the tracked entries; returns (batch positions, outputs [n, H_v, d_v])."""
        sel = self.entries(slot_ids)
        if len(sel) == 0:
            return sel, np.zeros((0,) + self.S.shape[1:2] + self.S.shape[3:])
        rows = np.array([self.row[int(slot_ids[e])] for e in sel])
        S_new, o = eager_step(self.S[rows], q[sel], a_or_k[sel], b_or_v[sel],
                              None if lam is None else lam[sel],
                              None if beta is None else beta[sel],
                              self.decay, self.update)
        self.S[rows] = S_new
        return sel, o

    def states(self, slots: Optional[Sequence[int]] = None) -> np.ndarray:
        if slots is None:
            return self.S
        return self.S[[self.row[int(s)] for s in slots]]


class RelL2:
    """Streaming relative L2 error ||x - ref|| / ||ref|| in float64."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.count = 0

    def add(self, x, ref) -> None:
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if x.shape != ref.shape:
            raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
        self.num += float(np.sum((x - ref) ** 2))
        self.den += float(np.sum(ref ** 2))
        self.count += ref.size

    @property
    def value(self) -> float:
        if self.den == 0.0:
            return 0.0 if self.num == 0.0 else float("inf")
        return float(np.sqrt(self.num / self.den))
