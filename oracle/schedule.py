"""Append/merge bookkeeping in closed form.

[DL] Algorithm 1 and the design section: with merge interval M (= L) and live
capacity C = M - 1, a cycle is C append steps followed by one merge step, after
which the log is empty.  [DL]'s allocator paragraph: a fresh or reused slot
starts with an empty log.  Counting decodes since a slot's last reset (fresh
assignment or explicit merge), with n0 live entries at that reset:

    live length before the j-th decode (j >= 1):  n = (n0 + j - 1) mod M
    the j-th decode merges                  iff   (n0 + j) mod M == 0
    otherwise it appends at log index n.

This module tracks only (n0, j) per slot and evaluates those two formulas; it
never increments or compares a counter the way the deferred pool does, so the
two can check each other.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np

APPEND, MERGE = 0, 1


def jth_decode(n0: int, M: int, j: int) -> Tuple[int, int]:
    """(phase, index) of the j-th decode since a reset with n0 live entries."""
    if j < 1:
        raise ValueError("j counts from 1")
    phase = MERGE if (n0 + j) % M == 0 else APPEND
    return phase, (n0 + j - 1) % M


class Counters:
    """Per-slot closed-form bookkeeping for a whole workload."""

    def __init__(self, num_slots: int, M: int):
        self.M = M
        self.n0 = np.zeros(num_slots, dtype=np.int64)
        self.j = np.zeros(num_slots, dtype=np.int64)
        self.merges = np.zeros(num_slots, dtype=np.int64)

    def reset(self, slots) -> None:
        """Fresh assignment: empty log."""
        for s in np.asarray(slots, dtype=np.int64):
            self.n0[s], self.j[s] = 0, 0

    def merge(self, slots) -> None:
        """Explicit materialization: the log becomes empty."""
        self.reset(slots)

    def decode(self, slots) -> List[Tuple[int, int]]:
        out = []
        for s in np.asarray(slots, dtype=np.int64):
            self.j[s] += 1
            ph = jth_decode(int(self.n0[s]), self.M, int(self.j[s]))
            if ph[0] == MERGE:
                self.merges[s] += 1
            out.append(ph)
        return out

    @property
    def n(self) -> np.ndarray:
        """Live-log length of every slot now."""
        return ((self.n0 + self.j) % self.M).astype(np.int64)
