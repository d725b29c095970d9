"""Seeded per-step input generation.

Every random draw comes from ``numpy.random.Generator(PCG64(key))`` with a key
that names what is drawn (workload seed, stream tag, step index, ...), so any
step, any slot's initial state and any replacement state can be regenerated on
its own, in any order, on any machine.  Stream tags:

  1  ragged-fill decode step (round r, chunk c)
  2  main decode step t
  3  initial base state of slot s
  4  fresh-state bank entry j
  5  initial log fill n0 of every slot
"""

from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .configs import Config


def round_to_bf16(x) -> np.ndarray:
    """float32 -> nearest-even bfloat16 value, returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _cast(x64: np.ndarray, dtype: str) -> np.ndarray:
    x = x64.astype(np.float32)
    if dtype == "bf16":
        x = round_to_bf16(x)
    elif dtype != "f32":
        raise ValueError(dtype)
    return x


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(k) for k in key]))


@dataclass(frozen=True)
class StepDesc:
    kind: str                     # "fill" | "main"
    index: tuple                  # fill: (round, chunk); main: (t,)
    slots: Optional[tuple] = None  # fill steps: the slots decoded


@dataclass
class StepInputs:
    desc: StepDesc
    slot_ids: np.ndarray          # int32 [B]
    q: np.ndarray                 # float32 [B, H_k, d]
    k: np.ndarray                 # float32 [B, H_k, d]   (a_t for plain operators)
    v: np.ndarray                 # float32 [B, H_v, d]   (b_t for plain operators)
    lam: Optional[np.ndarray]     # float32 [B, H_v] | [B, H_v, d] | None
    beta: Optional[np.ndarray]    # float32 [B, H_v] | None
    replace_ids: np.ndarray       # int32 [R]  slots given a fresh state before decoding
    replace_bank: np.ndarray      # int32 [R]  bank entry for each replaced slot

    @property
    def batch(self) -> int:
        return int(self.slot_ids.shape[0])


class Workload:
    """Deterministic input source for one :class:`Config`."""

    def __init__(self, cfg: Config):
        if cfg.H_v % cfg.H_k:
            raise ValueError("H_v must be a multiple of H_k")
        if cfg.replace_per_step > cfg.bank_size:
            raise ValueError("bank smaller than replacements per step")
        self.cfg = cfg

    # ---------------------------------------------------------------- schedule
    def initial_fill(self) -> np.ndarray:
        """Per-slot initial live-log length n0 (all zero unless ragged)."""
        c = self.cfg
        if not c.ragged_fill:
            return np.zeros(c.num_slots, dtype=np.int32)
        return _rng(c.seed, 5).integers(0, c.L, size=c.num_slots).astype(np.int32)

    def fill_steps(self) -> List[StepDesc]:
        """Decode steps that bring slot s to n0[s] live entries from empty.

        Round r decodes every slot with n0 > r, in chunks of at most B slots.
        """
        c = self.cfg
        n0 = self.initial_fill()
        out = []
        for r in range(c.L - 1):
            sl = np.nonzero(n0 > r)[0]
            for ci, lo in enumerate(range(0, len(sl), c.batch)):
                out.append(StepDesc("fill", (r, ci), tuple(int(s) for s in sl[lo:lo + c.batch])))
        return out

    def main_steps(self, steps: Optional[int] = None) -> List[StepDesc]:
        n = self.cfg.steps if steps is None else steps
        return [StepDesc("main", (t,)) for t in range(n)]

    def plan(self, steps: Optional[int] = None) -> List[StepDesc]:
        return self.fill_steps() + self.main_steps(steps)

    # ------------------------------------------------------------------ tokens
    def _tokens(self, rng: np.random.Generator, n: int):
        c = self.cfg
        shape_k = (n, c.H_k, c.d)
        shape_v = (n, c.H_v, c.d)
        if c.qk_dist == "unit":
            q = rng.standard_normal(shape_k)
            q /= np.linalg.norm(q, axis=-1, keepdims=True)
            k = rng.standard_normal(shape_k)
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
        elif c.qk_dist == "normal_scaled":
            q = rng.standard_normal(shape_k) * c.qk_scale
            k = rng.standard_normal(shape_k) * c.qk_scale
        else:
            raise ValueError(c.qk_dist)
        v = rng.standard_normal(shape_v) * c.v_scale
        lam = None
        if c.decay != "none":
            lshape = (n, c.H_v) if c.decay == "scalar" else (n, c.H_v, c.d)
            x = rng.normal(c.lam_mu, c.lam_sigma, size=lshape)
            lam = (-np.log1p(np.exp(-x))).astype(np.float32)     # logsigmoid
        beta = None
        if c.beta:
            x = rng.standard_normal((n, c.H_v))
            beta = (1.0 / (1.0 + np.exp(-x))).astype(np.float32)  # sigmoid
        return (_cast(q, c.in_dtype), _cast(k, c.in_dtype), _cast(v, c.in_dtype),
                lam, beta)

    def step_inputs(self, desc: StepDesc) -> StepInputs:
        c = self.cfg
        empty = np.zeros(0, dtype=np.int32)
        if desc.kind == "fill":
            rng = _rng(c.seed, 1, *desc.index)
            slots = np.asarray(desc.slots, dtype=np.int32)
            q, k, v, lam, beta = self._tokens(rng, len(slots))
            return StepInputs(desc, slots, q, k, v, lam, beta, empty, empty)
        if desc.kind != "main":
            raise ValueError(desc.kind)
        rng = _rng(c.seed, 2, *desc.index)
        rep_ids, rep_bank = empty, empty
        if c.replace_per_step:
            R = c.replace_per_step
            rep_ids = rng.choice(c.num_slots, size=R, replace=False).astype(np.int32)
            off = int(rng.integers(0, c.bank_size - R + 1))
            rep_bank = (off + np.arange(R)).astype(np.int32)
        if c.random_slots:
            slots = rng.choice(c.num_slots, size=c.batch, replace=False).astype(np.int32)
        else:
            slots = np.arange(c.batch, dtype=np.int32)
        q, k, v, lam, beta = self._tokens(rng, c.batch)
        return StepInputs(desc, slots, q, k, v, lam, beta, rep_ids, rep_bank)

    def generate(self, descs: Sequence[StepDesc], threads: Optional[int] = None) -> List[StepInputs]:
        """step_inputs over many steps, in parallel (each step has its own stream)."""
        threads = threads or min(16, os.cpu_count() or 1)
        if threads <= 1 or len(descs) < 4:
            return [self.step_inputs(d) for d in descs]
        with cf.ThreadPoolExecutor(threads) as ex:
            return list(ex.map(self.step_inputs, descs))

    # ------------------------------------------------------------------ states
    def _state(self, *key: int) -> np.ndarray:
        c = self.cfg
        if c.init_sigma == 0.0:
            return np.zeros((c.H_v, c.d, c.d), dtype=np.float32)
        x = _rng(*key).standard_normal((c.H_v, c.d, c.d), dtype=np.float32) * np.float32(c.init_sigma)
        return round_to_bf16(x) if c.state_dtype == "bf16" else x

    def _states(self, tag: int, ids: Sequence[int], threads: Optional[int]) -> np.ndarray:
        c = self.cfg
        ids = [int(i) for i in ids]
        out = np.empty((len(ids), c.H_v, c.d, c.d), dtype=np.float32)
        threads = threads or min(16, os.cpu_count() or 1)

        def one(j):
            out[j] = self._state(c.seed, tag, ids[j])

        if threads <= 1 or len(ids) < 4:
            for j in range(len(ids)):
                one(j)
        else:
            with cf.ThreadPoolExecutor(threads) as ex:
                list(ex.map(one, range(len(ids))))
        return out

    def init_base(self, slots: Optional[Sequence[int]] = None, threads: Optional[int] = None) -> np.ndarray:
        """Initial dense state of the given slots, float32 [n, H_v, d, d]."""
        if slots is None:
            slots = range(self.cfg.num_slots)
        return self._states(3, slots, threads)

    def bank_states(self, entries: Optional[Sequence[int]] = None, threads: Optional[int] = None) -> np.ndarray:
        """Fresh replacement states (bank entries), float32 [n, H_v, d, d]."""
        if entries is None:
            entries = range(self.cfg.bank_size)
        return self._states(4, entries, threads)
