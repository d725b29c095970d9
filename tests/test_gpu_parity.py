"""HIP path vs the fp64 oracle (E, the eager recurrence), through the C ABI.

Bar: outputs of every compared entry and final states rel-L2 <= 1e-4 (fp32
state) or 2e-2 (bf16 state); schedule, live-log counters (device and host) and
the lossless key-factor copies exact.
"""

import numpy as np
import pytest

from workloads import CONFIGS, headline_gdn, small_variant

pytestmark = pytest.mark.gpu


def _check(cfg, res):
    from gpu_harness import tolerance
    tol = tolerance(cfg)
    # every decoded entry of a tracked slot was compared, and some state
    assert res.compared_outputs == res.expected_outputs > 0
    assert res.compared_states > 0
    assert res.sched_mismatch == 0
    assert res.counter_mismatch == 0
    assert res.klog_mismatch == 0
    assert res.out_err <= tol, f"output rel-L2 {res.out_err:.3e} > {tol}"
    assert res.state_err <= tol, f"state rel-L2 {res.state_err:.3e} > {tol}"


# ---- the first two workloads at full size, every output compared
@pytest.mark.parametrize("idx", [1, 2])
def test_full_config(idx):
    from gpu_harness import run
    cfg = CONFIGS[idx]
    res = run(cfg)
    _check(cfg, res)
    assert res.merges == cfg.steps // cfg.L * cfg.batch


# ---- larger workloads at oracle-friendly sizes, every output compared
SMALL = {
    3: dict(batch=5, steps=96),
    4: dict(batch=7, steps=48),
    5: dict(num_slots=40, batch=13, steps=64, replace_per_step=2),
}


@pytest.mark.parametrize("idx", [3, 4, 5])
def test_small_config(idx):
    from gpu_harness import run
    cfg = small_variant(CONFIGS[idx], **SMALL[idx])
    _check(cfg, run(cfg))


# ---- full-size workloads in the launch configuration the benchmark times,
#      compared on a sample of slots followed by the oracle
TRACK = {3: [0, 31, 63], 4: [0, 77, 127], 5: [3, 100, 511, 777, 1023]}


@pytest.mark.parametrize("idx", [3, 4, 5])
def test_full_size_sampled(idx):
    """Every step of the workload as specified (512, 512 and 1024 steps; the
    serving pool's 1024 steps re-round its bf16 bases at every merge and at
    every one of its 52,224 replacements)."""
    from gpu_harness import run
    cfg = CONFIGS[idx]
    res = run(cfg, track=TRACK[idx])
    assert res.steps >= cfg.steps                 # main steps (plus the ragged fill's)
    _check(cfg, res)


@pytest.mark.parametrize("batch", [64, 256, 512])
def test_headline_gdn_batch_sampled(batch):
    """The GDN h32 d128 batch sweep the benchmark times, with its default
    whole-row tiles, on sampled slots."""
    from gpu_harness import run
    cfg = headline_gdn(batch, steps=64 if batch == 64 else 40)
    _check(cfg, run(cfg, track=[0, batch // 2 + 1, batch - 1]))


# ---- eager read-modify-write baseline kernel against the same oracle
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_eager_kernel(idx):
    from gpu_harness import run
    base = CONFIGS[idx]
    cfg = base if idx <= 2 else small_variant(base, **SMALL[idx])
    _check(cfg, run(cfg, eager=True))


# ---- every operator / dtype combination on small tiles (incl. the d = 16
#      bf16 tile whose row groups outnumber its rows), several merge intervals
COMBOS = [(decay, update, st, it)
          for decay in ("none", "scalar", "per_key")
          for update in ("plain", "delta")
          for st in ("f32", "bf16")
          for it in ("f32", "bf16")]


@pytest.mark.parametrize("d", [16, 32])
@pytest.mark.parametrize("combo", COMBOS, ids=lambda c: "-".join(c))
def test_operator_dtype_matrix(d, combo):
    from gpu_harness import run
    decay, update, st, it = combo
    cfg = small_variant(CONFIGS[4], batch=3, steps=23, L=5, d=d, H_v=4, H_k=2, decay=decay,
                        update=update, state_dtype=st, in_dtype=it,
                        name=f"matrix_d{d}_{decay}_{update}_{st}_{it}",
                        qk_dist="unit" if update == "delta" else "normal_scaled",
                        qk_scale=0.25, v_scale=1.0 if update == "delta" else 0.25,
                        lam_mu=None if decay == "none" else 3.0,
                        lam_sigma=None if decay == "none" else 1.0,
                        beta=update == "delta", init_sigma=0.02)
    _check(cfg, run(cfg))


@pytest.mark.parametrize("L", [1, 2, 3, 32, 64])
def test_merge_intervals(L):
    from gpu_harness import run
    cfg = small_variant(CONFIGS[4], batch=4, steps=2 * L + 3, L=L, d=64, H_v=4, H_k=4,
                        name=f"kda_L{L}")
    _check(cfg, run(cfg))


def test_explicit_merges_mid_stream():
    from gpu_harness import run
    cfg = small_variant(CONFIGS[2], steps=40, H_v=4, H_k=2, name="gdn_merge_every")
    _check(cfg, run(cfg, merge_every=3))


def test_batch_split_across_launches():
    """More decoded slots than one launch carries: the host splits the batch."""
    from gpu_harness import run
    import linear_attention_recurrent_dl_amd as dl
    lim = dl.dl_launch_slot_limit()
    cfg = small_variant(CONFIGS[1], batch=lim + 37, steps=10, L=4, d=16, H_v=2, H_k=1,
                        name="split_launch")
    _check(cfg, run(cfg, track=[0, lim - 1, lim, lim + 36]))


# ---- every built value-tile width (work units own d_k x B_V tiles)
TILES = [(128, 128), (128, 64), (128, 32), (128, 16), (64, 64), (64, 32)]


@pytest.mark.parametrize("d,bv", TILES)
@pytest.mark.parametrize("base_idx", [2, 3, 4, 5])
def test_value_tiles(d, bv, base_idx):
    from gpu_harness import run
    base = CONFIGS[base_idx]
    kw = dict(batch=3, steps=2 * base.L + 5, d=d, H_v=4, H_k=2 if base.H_k < base.H_v else 4,
              name=f"{base.name}_d{d}_bv{bv}")
    if base.random_slots:
        kw.update(num_slots=9, replace_per_step=1)
    cfg = small_variant(base, **kw)
    _check(cfg, run(cfg, value_tile=bv, merge_every=7))


@pytest.mark.parametrize("bv", [128, 64, 32, 16])
def test_value_tiles_headline_gdn(bv):
    """The batch-1 GDN workload at every tile width, every output compared."""
    from gpu_harness import run
    cfg = CONFIGS[2]
    _check(cfg, run(cfg, value_tile=bv))


# ---- split replay: ReplayPrep computes the key-side coefficients once per
#      (slot, v-head) into the scratch, the appending tile units read them
#      ([DL] GPU-execution section); merging slots still replay in-block
@pytest.mark.parametrize("combo", COMBOS, ids=lambda c: "-".join(c))
def test_split_replay_operator_dtype_matrix(combo):
    from gpu_harness import run
    decay, update, st, it = combo
    cfg = small_variant(CONFIGS[4], batch=3, steps=23, L=5, d=64, H_v=4, H_k=2, decay=decay,
                        update=update, state_dtype=st, in_dtype=it,
                        name=f"split_matrix_{decay}_{update}_{st}_{it}",
                        qk_dist="unit" if update == "delta" else "normal_scaled",
                        qk_scale=0.25, v_scale=1.0 if update == "delta" else 0.25,
                        lam_mu=None if decay == "none" else 3.0,
                        lam_sigma=None if decay == "none" else 1.0,
                        beta=update == "delta", init_sigma=0.02)
    _check(cfg, run(cfg, value_tile=32, replay_split=True))


@pytest.mark.parametrize("d,bv", [(128, 128), (128, 64), (128, 32), (128, 16), (64, 64), (64, 32)])
@pytest.mark.parametrize("base_idx", [2, 3, 4, 5])
def test_split_replay_value_tiles(d, bv, base_idx):
    from gpu_harness import run
    base = CONFIGS[base_idx]
    kw = dict(batch=3, steps=2 * base.L + 5, d=d, H_v=4, H_k=2 if base.H_k < base.H_v else 4,
              name=f"split_{base.name}_d{d}_bv{bv}")
    if base.random_slots:
        kw.update(num_slots=9, replace_per_step=1)
    cfg = small_variant(base, **kw)
    _check(cfg, run(cfg, value_tile=bv, merge_every=7, replay_split=True))


def test_split_replay_headline_gdn():
    """The batch-1 GDN workload, 32-column tiles (four per head), every output compared."""
    from gpu_harness import run
    cfg = CONFIGS[2]
    _check(cfg, run(cfg, value_tile=32, replay_split=True))


# ---- edge shapes: the longest log (63 live entries, past the up-front
#      prefetch, so the remainder staging loop runs) at d = 128, and eight
#      v-heads sharing one q/k head (one designated key writer per group)
@pytest.mark.parametrize("base_idx,bv", [(2, 64), (2, 32), (4, 64)])
def test_longest_log_d128(base_idx, bv):
    from gpu_harness import run
    base = CONFIGS[base_idx]
    cfg = small_variant(base, batch=2, steps=140, L=64 if base.decay != "per_key" else 32, d=128, H_v=4,
                        H_k=2 if base.H_k < base.H_v else 4, name=f"longlog_{base.name}_bv{bv}")
    _check(cfg, run(cfg, value_tile=bv))


def test_longest_per_key_log_default_tile():
    """KDA-style at d = 128 with L = 64 and 256 slot-heads per launch: the
    whole-row default tile's 63 live entries (bf16 keys, fp32 values, per-key
    snapshots) would need 80,640 B of LDS, so the default falls back to 32
    columns (56,448 B, just inside the budget)."""
    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import run
    cfg = small_variant(CONFIGS[4], batch=64, num_slots=64, steps=140, L=64, d=128, H_v=4, H_k=4,
                        name="longlog_kda_L64_default_tile")
    desc = dl.make_desc(cfg.num_slots, cfg.batch, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update,
                        cfg.state_dtype, cfg.in_dtype)
    assert dl.dl_value_tile(desc) == 32
    _check(cfg, run(cfg, track=[0, 21, 63]))


@pytest.mark.parametrize("split", [False, True])
def test_eight_v_heads_per_qk_head(split):
    from gpu_harness import run
    cfg = small_variant(CONFIGS[2], batch=3, steps=37, L=6, d=64, H_v=16, H_k=2, name="gva8")
    _check(cfg, run(cfg, value_tile=32, replay_split=split))
