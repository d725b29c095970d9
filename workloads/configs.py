"""The five decode workloads, as data.

Operator families follow the DeltaLog paper ("DeltaLog: Deferred Materialization
of Recurrent States for Linear Attention Decoding"), Table 1 and the operator
instantiations section: plain linear attention (no decay), GDN (head-wise scalar
decay + delta rule), GLA/RWKV6-style (per-key decay, raw value) and KDA
(per-key decay + delta rule).  Grouped value heads (two v-heads per q/k head)
follow the FPGA GDN-decode paper ("A Persistent-State Dataflow Accelerator for
Memory-Bound Linear Attention Decode on FPGA"), system architecture / Table II.

Readings where the workload text leaves a choice open are listed in the
project's design notes; the ones that shape data here are:
  * N(mu, s): s is a standard deviation.
  * GDN "32 value heads" use 16 q/k heads (the FPGA paper's Table II token I/O
    of 49,664 B only adds up with 16 q/k heads).
  * A single input dtype covers q, k (or a) and v (or b).  The GLA-style
    workload stores bf16 factors with a = k and b = v, so its q, k, v are bf16.
  * Unstated initial bases of the GLA and KDA workloads are N(0, 0.02).
  * The serving pool replaces floor(5% * 1024) = 51 slots per step.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    decay: str              # "none" | "scalar" | "per_key"
    update: str             # "plain" | "delta"
    num_slots: int          # pool size P
    batch: int              # decoded entries per step B
    H_v: int                # value heads
    H_k: int                # query/key heads (H_v % H_k == 0)
    d: int                  # d_k == d_v
    state_dtype: str        # "f32" | "bf16"  (dense base)
    in_dtype: str           # "f32" | "bf16"  (q, k/a, v/b)
    L: int                  # merge interval (log capacity L - 1)
    steps: int              # main decode steps
    init_sigma: float       # 0.0 = zero initial state
    seed: int
    # token-input distributions
    qk_dist: str            # "normal_scaled" | "unit"   (unit = L2-normalised N(0,1))
    qk_scale: float         # scale for "normal_scaled"
    v_scale: float          # v (or b) ~ N(0, 1) * v_scale
    lam_mu: Optional[float] = None      # log-decay = logsigmoid(N(lam_mu, lam_sigma))
    lam_sigma: Optional[float] = None
    beta: bool = False                  # beta = sigmoid(N(0, 1)) when True
    # serving-pool behaviour
    random_slots: bool = False          # B distinct random slot ids per step
    replace_per_step: int = 0           # fresh states assigned before each step
    ragged_fill: bool = False           # initial log fill n0 ~ U{0..L-1} per slot
    bank_size: int = 64                 # distinct fresh states to draw replacements from

    @property
    def gva(self) -> int:
        return self.H_v // self.H_k

    def describe(self) -> str:
        return (f"{self.name}: P={self.num_slots} B={self.batch} H_v={self.H_v} "
                f"H_k={self.H_k} d={self.d} {self.decay}/{self.update} "
                f"state={self.state_dtype} in={self.in_dtype} L={self.L} "
                f"steps={self.steps}")


_C = {}


def _add(cfg: Config) -> None:
    _C[cfg.index] = cfg


# 1. Plain linear attention: lambda = 0, b_t given, zero state.
_add(Config(index=1, name="plain_la_b1_h2_d16", decay="none", update="plain",
            num_slots=1, batch=1, H_v=2, H_k=2, d=16, state_dtype="f32",
            in_dtype="f32", L=8, steps=64, init_sigma=0.0, seed=1001,
            qk_dist="normal_scaled", qk_scale=0.25, v_scale=0.25))

# 2. Gated DeltaNet decode at batch 1 (32 v-heads, 16 q/k heads, 2 MiB fp32 state).
_add(Config(index=2, name="gdn_b1_h32_d128", decay="scalar", update="delta",
            num_slots=1, batch=1, H_v=32, H_k=16, d=128, state_dtype="f32",
            in_dtype="f32", L=16, steps=256, init_sigma=0.02, seed=1002,
            qk_dist="unit", qk_scale=1.0, v_scale=1.0, lam_mu=3.0,
            lam_sigma=0.5, beta=True))

# 3. Diagonal-decay GLA / RWKV6-style (raw value), bf16 factors.
_add(Config(index=3, name="gla_b64_h32_d64", decay="per_key", update="plain",
            num_slots=64, batch=64, H_v=32, H_k=32, d=64, state_dtype="f32",
            in_dtype="bf16", L=32, steps=512, init_sigma=0.02, seed=1003,
            qk_dist="normal_scaled", qk_scale=0.125, v_scale=0.125,
            lam_mu=4.0, lam_sigma=1.0))

# 4. Kimi-Delta-style: per-key decay + delta rule, bf16 q/k/v.
_add(Config(index=4, name="kda_b128_h32_d128", decay="per_key", update="delta",
            num_slots=128, batch=128, H_v=32, H_k=32, d=128, state_dtype="f32",
            in_dtype="bf16", L=16, steps=512, init_sigma=0.02, seed=1004,
            qk_dist="unit", qk_scale=1.0, v_scale=1.0, lam_mu=3.0,
            lam_sigma=1.0, beta=True))

# 5. Serving pool: 1024 bf16 slots, GDN grouped heads, 256 random slots per step.
_add(Config(index=5, name="gdn_pool1024_b256_h32_d128_bf16", decay="scalar",
            update="delta", num_slots=1024, batch=256, H_v=32, H_k=16, d=128,
            state_dtype="bf16", in_dtype="bf16", L=16, steps=1024,
            init_sigma=0.02, seed=1005, qk_dist="unit", qk_scale=1.0,
            v_scale=1.0, lam_mu=3.0, lam_sigma=0.5, beta=True,
            random_slots=True, replace_per_step=51, ragged_fill=True))

CONFIGS = dict(_C)


def headline_gdn(batch: int, L: int = 16, steps: int = 256, seed: int = 1100) -> Config:
    """GDN fp32, 32 v-heads / 16 q/k heads, d = 128 at a given batch.

    The DeltaLog paper's kernel evaluation sweeps B in {64, 128, 256, 512} for
    this operator family; this is that shape on one pool of B slots.
    """
    base = CONFIGS[2]
    return dataclasses.replace(base, index=100 + batch, name=f"gdn_b{batch}_h32_d128",
                               num_slots=batch, batch=batch, L=L, steps=steps,
                               seed=seed + batch)


def at_batch(cfg: Config, batch: int, steps: Optional[int] = None) -> Config:
    """A fixed-slot workload (configs 3 and 4) at another batch: B slots, all
    decoded every step, same operator, dtypes and distributions."""
    return dataclasses.replace(cfg, index=cfg.index * 1000 + batch,
                               name=cfg.name.replace(f"_b{cfg.batch}_", f"_b{batch}_"), num_slots=batch,
                               batch=batch, steps=cfg.steps if steps is None else steps, seed=cfg.seed + batch)


SWEEP_OPERATORS = ("plain", "gdn", "gla", "kda")


def merge_sweep_config(op: str, L: int, batch: int = 128) -> Config:
    """One operator family at batch B, 32 v-heads, d = 128, fp32 state, merge
    interval L: the shapes of the DeltaLog paper's merge-interval sweep (its
    kernel-evaluation section sweeps M at B = 128 per operator).  Inputs keep
    each family's workload distributions and dtypes above."""
    if op == "gdn":
        return dataclasses.replace(headline_gdn(batch, L=L), name=f"gdn_b{batch}_h32_d128_L{L}")
    src = {"plain": CONFIGS[1], "gla": CONFIGS[3], "kda": CONFIGS[4]}[op]
    kw = dict(index=200 + batch, name=f"{op}_b{batch}_h32_d128_L{L}", num_slots=batch, batch=batch,
              H_v=32, d=128, L=L, steps=256, seed=src.seed + 7 * L)
    if op == "plain":
        kw.update(H_k=32, init_sigma=0.02)
    if op == "gla":
        kw.update(H_k=32)
    return dataclasses.replace(src, **kw)


def get_config(index: int) -> Config:
    return CONFIGS[index]


def small_variant(cfg: Config, *, batch: Optional[int] = None,
                  num_slots: Optional[int] = None, steps: Optional[int] = None,
                  replace_per_step: Optional[int] = None, L: Optional[int] = None,
                  seed_offset: int = 0, **kw) -> Config:
    """Same operator, dtypes and distributions at an oracle-friendly size."""
    ch = {}
    if batch is not None:
        ch["batch"] = batch
        if not cfg.random_slots and num_slots is None:
            ch["num_slots"] = batch
    if num_slots is not None:
        ch["num_slots"] = num_slots
    if steps is not None:
        ch["steps"] = steps
    if replace_per_step is not None:
        ch["replace_per_step"] = replace_per_step
    if L is not None:
        ch["L"] = L
    ch["seed"] = cfg.seed + seed_offset
    ch.update(kw)
    ch.setdefault("name", cfg.name + "_small")
    return dataclasses.replace(cfg, **ch)


def shape_tuple(cfg: Config) -> Tuple[int, int, int, int]:
    return (cfg.num_slots, cfg.H_v, cfg.d, cfg.d)
