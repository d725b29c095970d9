"""Algorithmic HBM bytes of one decode step, per (slot, v-head).

This is the recurrent-state traffic model that the DeltaLog paper names
(C_log(M), design section) but whose formula did not survive, rebuilt from its
physical-state list for this library's storage layout:

  base      d_k * d_v * s_state                   read every step, written at a merge
  entry E   d_k * s_a * H_k / H_v                 key factor (one per q/k head, shared
            + d_v * s_b                           by the v-heads of a group)
            + |Lambda| (4 B scalar or 4 * d_k)    value factor and decay snapshot
  tokens    q, k: d_k * s_in * H_k / H_v each; v: d_v * s_in; lambda; beta
  output    4 * d_v
  counter   4 B read + 4 B written (live-log length)

A step with n live entries reads n entries; an append writes one entry, a
merge writes the base instead.  The eager read-modify-write baseline reads and
writes the base every step and has no log.  The cumulative log-decay is not
stored: it equals the newest entry's snapshot (or 0 for an empty log).

The FPGA paper "A Persistent-State Dataflow Accelerator for Memory-Bound
Linear Attention Decode on FPGA" prints, in Table II, the eager state I/O of a
32-head d = 128 fp32 GDN token (4,194,304 B) and its token I/O (49,664 B);
``eager_state_bytes`` and ``token_bytes`` reproduce both.
"""

from __future__ import annotations

from dataclasses import dataclass

DTYPE_BYTES = {"f32": 4, "bf16": 2}


def eager_state_bytes(H_v: int, d_k: int, d_v: int, state_bytes: int) -> int:
    """Dense state read + write per token, all v-heads."""
    return 2 * H_v * d_k * d_v * state_bytes


def token_bytes(H_v: int, H_k: int, d_k: int, d_v: int, in_bytes: int,
                per_head_scalars: int, out_bytes: int = 4) -> int:
    """q and k per q/k head, v and o per v-head, plus fp32 per-v-head scalars."""
    return (2 * H_k * d_k * in_bytes + H_v * d_v * in_bytes + H_v * d_v * out_bytes
            + 4 * per_head_scalars * H_v)


@dataclass(frozen=True)
class StepShape:
    H_v: int
    H_k: int
    d_k: int
    d_v: int
    decay: str          # "none" | "scalar" | "per_key"
    update: str         # "plain" | "delta"
    state_dtype: str    # "f32" | "bf16"
    in_dtype: str       # "f32" | "bf16"
    L: int

    @property
    def s_state(self) -> int:
        return DTYPE_BYTES[self.state_dtype]

    @property
    def s_in(self) -> int:
        return DTYPE_BYTES[self.in_dtype]

    @property
    def s_b(self) -> int:
        return 4 if self.update == "delta" else self.s_in

    @property
    def lam_bytes(self) -> int:
        return {"none": 0, "scalar": 4, "per_key": 4 * self.d_k}[self.decay]

    @property
    def base_bytes(self) -> int:
        return self.d_k * self.d_v * self.s_state

    @property
    def entry_bytes(self) -> float:
        snap = 0 if self.decay == "none" else self.lam_bytes
        return self.d_k * self.s_in * self.H_k / self.H_v + self.d_v * self.s_b + snap

    @property
    def token_io(self) -> float:
        qk = 2 * self.d_k * self.s_in * self.H_k / self.H_v
        beta = 4 if self.update == "delta" else 0
        return qk + self.d_v * self.s_in + self.lam_bytes + beta + 4 * self.d_v


def deltalog_head_step_bytes(sh: StepShape, n: int) -> float:
    """One (slot, v-head) decode with n live entries (merge iff n == L - 1)."""
    merge = n == sh.L - 1
    b = sh.base_bytes + n * sh.entry_bytes + sh.token_io + 8
    b += sh.base_bytes if merge else sh.entry_bytes
    return b


def deltalog_model_bytes(sh: StepShape) -> float:
    """Average over a full cycle (n uniform on 0..L-1)."""
    return sum(deltalog_head_step_bytes(sh, n) for n in range(sh.L)) / sh.L


def eager_head_step_bytes(sh: StepShape) -> float:
    return 2 * sh.base_bytes + sh.token_io


def merge_head_bytes(sh: StepShape, n: int) -> float:
    """Standalone materialization of n live entries (no token)."""
    if n == 0:
        return 4.0
    return 2 * sh.base_bytes + n * sh.entry_bytes + 8


def assign_head_bytes(sh: StepShape, zero: bool = False) -> float:
    """Fresh-slot assignment: copy (or zero) the base, clear the counter."""
    return (sh.base_bytes if zero else 2 * sh.base_bytes) + 4


def window_head_bytes(sh: StepShape, W: int, n: int = 0) -> float:
    """One (slot, v-head) over a window of W steps held on chip: the base and
    n live entries read once, the base written once, W steps of token I/O,
    the counter read and cleared."""
    return 2 * sh.base_bytes + n * sh.entry_bytes + W * sh.token_io + 8
