"""Decode steps captured in a HIP graph and replayed, against the fp64 oracle.

The decode kernel reads each slot-head's live-log length on the device, so a
captured sequence of steps (append and merge alike) stays valid for every
replay: replay r applies the same token inputs again to the state the previous
replay left.  Each replay is checked against the oracle, with eager device work
and synchronizations between replays.
"""

import numpy as np
import pytest

from workloads import CONFIGS, Workload, small_variant

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx,value_tile,split", [(2, 0, False), (2, 32, False), (4, 0, False), (5, 0, False),
                                                 (2, 32, True), (4, 32, True)])
def test_graph_replay_matches_oracle(idx, value_tile, split):
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    base = CONFIGS[idx]
    kw = dict(batch=3, steps=6, H_v=4, H_k=2 if base.H_k < base.H_v else 4, L=4,
              name=f"graph_{base.name}", random_slots=False, replace_per_step=0, ragged_fill=False)
    if base.random_slots:
        kw["num_slots"] = 3
    cfg = small_variant(base, **kw)
    say(f"[gpu] graph replay {cfg.describe()} value_tile={value_tile} replay_split={split}")
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    P = cfg.num_slots
    pool = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, max_batch=cfg.batch, value_tile=value_tile, replay_split=split)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    dev = [dict(q=to_dev(s.q, it), k=to_dev(s.k, it), v=to_dev(s.v, it),
                lam=to_dev(s.lam, torch.float32), beta=to_dev(s.beta, torch.float32),
                out=torch.empty((cfg.batch, cfg.H_v, cfg.d), dtype=torch.float32, device="cuda"))
           for s in steps]
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s, d in zip(steps, dev):
            pool.decode_step(s.slot_ids, d["q"], d["k"], d["v"], d["lam"], d["beta"], d["out"])
    # capture launched nothing: the state is still the initial one
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        err = RelL2()
        for s, d in zip(steps, dev):
            _, o_ref = E.step(s.slot_ids, s.q, s.k, s.v, s.lam, s.beta)
            err.add(d["out"].cpu().numpy(), o_ref)
        scratch.mul_(0.5).add_(1.0)              # unrelated eager work between replays
        torch.cuda.synchronize()
        n_dev = pool.device_log_len()
        want_n = ((rep + 1) * cfg.steps) % cfg.L
        say(f"[gpu]   replay {rep}: out rel-L2 {err.value:.3e}, device n {sorted(set(n_dev.ravel().tolist()))}")
        tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
        assert err.value <= tol
        assert np.all(n_dev == want_n)
    pool.close()


@pytest.mark.parametrize("idx,nsteps", [(2, 14), (4, 14), (5, 14), (2, 12), (5, 12)])
def test_direct_steps_after_a_capture(idx, nsteps):
    """Capturing steps advances the host's live lengths but not the device's.
    Direct steps afterwards carry host values that differ from the device
    counters, so every block restages its log from the counter; outputs,
    states and device counters must follow the direct steps alone.  With 12
    steps (3 captured, 9 direct, L = 4) the host mirror ends at 0 while every
    device log holds 1 entry: dl_flush_all must still merge it."""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2, schedule

    base = CONFIGS[idx]
    cfg = small_variant(base, batch=3, steps=nsteps, H_v=4, H_k=2 if base.H_k < base.H_v else 4, L=4,
                        name=f"capture_then_direct_{base.name}", random_slots=False, replace_per_step=0,
                        ragged_fill=False, num_slots=3)
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    P = cfg.num_slots
    pool = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, max_batch=cfg.batch)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
    cnt = schedule.Counters(P, cfg.L)
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    dev = [dict(q=to_dev(s.q, it), k=to_dev(s.k, it), v=to_dev(s.v, it), lam=to_dev(s.lam, torch.float32),
                beta=to_dev(s.beta, torch.float32)) for s in steps]
    say(f"[gpu] direct steps after a capture: {cfg.describe()}")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):                  # recorded, never replayed
        for s, d in zip(steps[:3], dev[:3]):
            pool.decode_step(s.slot_ids, d["q"], d["k"], d["v"], d["lam"], d["beta"])
    torch.cuda.synchronize()
    assert np.all(pool.log_len() == 3) and np.all(pool.device_log_len() == 0)
    err = RelL2()
    for s, d in zip(steps[3:], dev[3:]):
        out = pool.decode_step(s.slot_ids, d["q"], d["k"], d["v"], d["lam"], d["beta"])
        _, o_ref = E.step(s.slot_ids, s.q, s.k, s.v, s.lam, s.beta)
        cnt.decode(s.slot_ids)
        err.add(out.cpu().numpy(), o_ref)
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len() == cnt.n[:, None])
    assert np.all(pool.log_len() == nsteps % cfg.L)     # the mirror counts the captured calls too
    pool.flush_all()
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len() == 0)
    st_e = RelL2()
    st_e.add(pool.read_base(ids).float().cpu().numpy(), E.states())
    tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
    say(f"[gpu]   out rel-L2 {err.value:.3e}, state rel-L2 {st_e.value:.3e}")
    del g
    pool.close()
    assert err.value <= tol and st_e.value <= tol


@pytest.mark.parametrize("idx", [2, 5])
def test_merge_recorded_in_a_graph(idx):
    """dl_merge recorded into a graph: its launch covers the listed slots, and
    each block merges whatever its device counter holds at replay (nothing
    when empty).  Slots outside the recorded set keep their logs; every state
    and counter follows the oracle."""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    base = CONFIGS[idx]
    cfg = small_variant(base, batch=4, steps=8, H_v=4, H_k=2 if base.H_k < base.H_v else 4, L=4,
                        name=f"graph_merge_{base.name}", random_slots=False, replace_per_step=0,
                        ragged_fill=False, num_slots=4)
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    P = cfg.num_slots
    pool = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, max_batch=P)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
    err = RelL2()

    def step(s):
        out = pool.decode_step(s.slot_ids, to_dev(s.q, it), to_dev(s.k, it), to_dev(s.v, it),
                               to_dev(s.lam, torch.float32), to_dev(s.beta, torch.float32))
        _, o_ref = E.step(s.slot_ids, s.q, s.k, s.v, s.lam, s.beta)
        err.add(out.cpu().numpy(), o_ref)

    def states_match(slots):
        e = RelL2()
        e.add(pool.read_base(slots).float().cpu().numpy(), E.states(slots))
        return e.value

    say(f"[gpu] merge recorded in a graph: {cfg.describe()}")
    step(steps[0])
    step(steps[1])                                # every slot holds 2 entries
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pool.merge(np.array([0, 1], dtype=np.int32))
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len() == 2)     # recorded, not run
    g.replay()
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len()[:2] == 0) and np.all(pool.device_log_len()[2:] == 2)
    assert states_match([0, 1]) <= tol            # their logs are in the bases now
    g.replay()                                    # empty logs: every block exits at once
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len()[:2] == 0) and states_match([0, 1]) <= tol
    step(steps[2])                                # host and device agree again: 1, 1, 3, 3
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len() == np.array([1, 1, 3, 3])[:, None])
    g.replay()                                    # merges the single entries of slots 0 and 1
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len() == np.array([0, 0, 3, 3])[:, None])
    assert states_match([0, 1]) <= tol
    pool.flush_all()                              # mirror stale since the capture: every slot is launched
    torch.cuda.synchronize()
    assert np.all(pool.device_log_len() == 0)
    st_all = states_match(ids)
    say(f"[gpu]   out rel-L2 {err.value:.3e}, state rel-L2 {st_all:.3e}")
    del g
    pool.close()
    assert err.value <= tol and st_all <= tol


@pytest.mark.parametrize("idx", [2, 5])
def test_flush_after_replays_the_mirror_missed(idx):
    """Two direct steps, then two steps captured and replayed twice (L = 4):
    the host mirror reads 0 entries, every device log holds 2.  dl_flush_all
    (and dl_merge) must materialize those logs: the bases then equal the
    oracle's states after all six decodes, and every counter reads 0."""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    base = CONFIGS[idx]
    cfg = small_variant(base, batch=3, steps=4, H_v=4, H_k=2 if base.H_k < base.H_v else 4, L=4,
                        name=f"replays_then_flush_{base.name}", random_slots=False, replace_per_step=0,
                        ragged_fill=False, num_slots=3)
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    P = cfg.num_slots
    tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
    for how in ("flush_all", "merge"):
        say(f"[gpu] replays the mirror missed, then {how}: {cfg.describe()}")
        pool = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype,
                               cfg.in_dtype, max_batch=cfg.batch)
        ids = np.arange(P, dtype=np.int32)
        pool.assign(ids, to_dev(wl.init_base(ids), st))
        E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
        steps = [wl.step_inputs(d) for d in wl.main_steps()]
        dev = [dict(q=to_dev(s.q, it), k=to_dev(s.k, it), v=to_dev(s.v, it), lam=to_dev(s.lam, torch.float32),
                    beta=to_dev(s.beta, torch.float32)) for s in steps]
        for s, d in zip(steps[:2], dev[:2]):
            pool.decode_step(s.slot_ids, d["q"], d["k"], d["v"], d["lam"], d["beta"])
            E.step(s.slot_ids, s.q, s.k, s.v, s.lam, s.beta)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s, d in zip(steps[2:], dev[2:]):
                pool.decode_step(s.slot_ids, d["q"], d["k"], d["v"], d["lam"], d["beta"])
        for _ in range(2):
            g.replay()
            torch.cuda.synchronize()
            for s in steps[2:]:
                E.step(s.slot_ids, s.q, s.k, s.v, s.lam, s.beta)
        assert np.all(pool.log_len() == 0) and np.all(pool.device_log_len() == 2)
        if how == "flush_all":
            pool.flush_all()
        else:
            pool.merge(ids)
        torch.cuda.synchronize()
        n_dev = pool.device_log_len()
        e = RelL2()
        e.add(pool.read_base(ids).float().cpu().numpy(), E.states())
        say(f"[gpu]   state rel-L2 {e.value:.3e}, device n {sorted(set(n_dev.ravel().tolist()))}")
        del g
        pool.close()
        assert np.all(n_dev == 0)
        assert e.value <= tol


def test_serving_pool_steps_with_assignments_in_a_graph():
    """The serving pool's step as the benchmark records it: fresh-state
    assignments, then the decode of random slots, several steps captured in
    one graph and replayed three times.  Every replay re-assigns the same
    fresh states and decodes the same tokens; outputs after each replay and
    the final states follow the oracle."""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    cfg = small_variant(CONFIGS[5], batch=4, num_slots=9, steps=6, H_v=4, H_k=2, L=4, replace_per_step=2,
                        ragged_fill=False, bank_size=8, name="graph_pool_assign")
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    P = cfg.num_slots
    pool = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, max_batch=P)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
    bank = wl.bank_states()
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    assert all(len(s.replace_ids) == 2 for s in steps)
    dev = [dict(init=to_dev(bank[s.replace_bank], st), q=to_dev(s.q, it), k=to_dev(s.k, it), v=to_dev(s.v, it),
                lam=to_dev(s.lam, torch.float32), beta=to_dev(s.beta, torch.float32),
                out=torch.empty((cfg.batch, cfg.H_v, cfg.d), dtype=torch.float32, device="cuda"))
           for s in steps]
    say(f"[gpu] serving-pool steps with assignments in a graph: {cfg.describe()}")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s, d in zip(steps, dev):
            pool.assign(s.replace_ids, d["init"])
            pool.decode_step(s.slot_ids, d["q"], d["k"], d["v"], d["lam"], d["beta"], d["out"])
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        err = RelL2()
        for s, d in zip(steps, dev):
            E.assign(s.replace_ids, bank[s.replace_bank])
            _, o_ref = E.step(s.slot_ids, s.q, s.k, s.v, s.lam, s.beta)
            err.add(d["out"].cpu().numpy(), o_ref)
        scratch.mul_(0.5).add_(1.0)
        torch.cuda.synchronize()
        say(f"[gpu]   replay {rep}: out rel-L2 {err.value:.3e}")
        assert err.value <= 2e-2
    pool.flush_all()
    st_e = RelL2()
    st_e.add(pool.read_base(ids).float().cpu().numpy(), E.states())
    say(f"[gpu]   state rel-L2 {st_e.value:.3e}")
    del g
    pool.close()
    assert st_e.value <= 2e-2


@pytest.mark.parametrize("idx,L,value_tile,in_dtype", [(2, 4, 128, None), (5, 4, 128, None), (3, 4, 0, None),
                                                          (4, 4, 0, None), (5, 4, 0, None), (4, 1, 0, None),
                                                          (2, 1, 128, None), (1, 4, 0, "bf16")])
def test_consecutive_and_gathered_slots(idx, L, value_tile, in_dtype):
    """Launches whose slots are consecutive name their first slot instead of
    carrying slot words (the blocks then compute their slots).  Consecutive
    runs that start past slot 0, gathered sets and single slots, decoded
    directly and from a replayed graph, merged and flushed, all follow the
    oracle; L = 1 runs the eager kernel through the same launches.  (Plain LA
    at d = 16 with bf16 inputs has two key chunks per entry, too few for the
    one-barrier narrow kernel: it runs the narrow-tile staging of the general
    decode kernel.)"""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    base = CONFIGS[idx]
    extra = {"in_dtype": in_dtype} if in_dtype else {}
    cfg = small_variant(base, batch=3, steps=6, H_v=4, H_k=2 if base.H_k < base.H_v else 4, L=L,
                        name=f"consecutive_{base.name}", random_slots=False, replace_per_step=0,
                        ragged_fill=False, num_slots=10, **extra)
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    P = cfg.num_slots
    pool = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, max_batch=P, value_tile=value_tile)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
    sets = [np.array(s, dtype=np.int32) for s in ([4, 5, 6], [8, 1, 5], [7, 8, 9], [2, 3, 4], [6, 0, 9])]
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
    say(f"[gpu] consecutive / gathered slots: {cfg.describe()} value_tile={value_tile}")
    err = RelL2()
    step_fn = pool.eager_step if L == 1 else pool.decode_step

    def run(s, slots, out=None, check=True):
        o = step_fn(slots, to_dev(s.q, it), to_dev(s.k, it), to_dev(s.v, it),
                    to_dev(s.lam, torch.float32), to_dev(s.beta, torch.float32), out)
        if check:
            _, o_ref = E.step(slots, s.q, s.k, s.v, s.lam, s.beta)
            err.add(o.cpu().numpy(), o_ref)
        return o

    for k, s in enumerate(steps):                  # direct launches
        run(s, sets[k % len(sets)])
    torch.cuda.synchronize()
    say(f"[gpu]   direct: out rel-L2 {err.value:.3e}")
    # captured: one step per slot set, then replayed with checks between
    dev = [dict(q=to_dev(s.q, it), k=to_dev(s.k, it), v=to_dev(s.v, it), lam=to_dev(s.lam, torch.float32),
                beta=to_dev(s.beta, torch.float32),
                out=torch.empty((cfg.batch, cfg.H_v, cfg.d), dtype=torch.float32, device="cuda"))
           for s in steps[:len(sets)]]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d, slots in zip(dev, sets):
            step_fn(slots, d["q"], d["k"], d["v"], d["lam"], d["beta"], d["out"])
        if L > 1:
            pool.merge(np.array([7, 8, 9], dtype=np.int32))
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for s, d, slots in zip(steps, dev, sets):
            _, o_ref = E.step(slots, s.q, s.k, s.v, s.lam, s.beta)
            err.add(d["out"].cpu().numpy(), o_ref)
        say(f"[gpu]   replay {rep}: out rel-L2 {err.value:.3e}")
    if L > 1:
        n_dev = pool.device_log_len()
        assert np.all(n_dev[7:10] == 0)            # the recorded merge emptied them at every replay
    pool.flush_all()
    torch.cuda.synchronize()
    se = RelL2()
    se.add(pool.read_base(ids).float().cpu().numpy(), E.states(ids))
    say(f"[gpu]   out rel-L2 {err.value:.3e}, state rel-L2 {se.value:.3e}")
    del g
    pool.close()
    assert err.value <= tol and se.value <= tol


def test_consecutive_slots_split_over_launches():
    """A recorded call over more slots than one launch carries is split into
    launches, each of which decides on its own whether its slots are
    consecutive: a run of 1100 slots (three consecutive launches, the second
    and third starting past slot 0) and a gathered permutation of the same
    slots, replayed, against the oracle (plain LA, d = 16, L = 4, bf16 inputs:
    the general decode kernel, which takes the first slot of a consecutive
    launch)."""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    base = CONFIGS[1]
    P = 1100
    cfg = small_variant(base, batch=P, steps=4, L=4, name="consecutive_split", num_slots=P, in_dtype="bf16")
    assert dl.dl_launch_slot_limit() < P
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    pool = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, max_batch=P)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
    perm = np.random.default_rng(7).permutation(P).astype(np.int32)
    sets = [ids, perm, ids, perm]
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    say(f"[gpu] consecutive launches split: {cfg.describe()}")
    dev = [dict(q=to_dev(s.q, it), k=to_dev(s.k, it), v=to_dev(s.v, it),
                out=torch.empty((P, cfg.H_v, cfg.d), dtype=torch.float32, device="cuda")) for s in steps]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d, slots in zip(dev, sets):
            pool.decode_step(slots, d["q"], d["k"], d["v"], None, None, d["out"])
    torch.cuda.synchronize()
    err = RelL2()
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        for s, d, slots in zip(steps, dev, sets):
            _, o_ref = E.step(slots, s.q, s.k, s.v, None, None)
            err.add(d["out"].cpu().numpy(), o_ref)
    pool.flush_all()
    torch.cuda.synchronize()
    se = RelL2()
    se.add(pool.read_base(ids).float().cpu().numpy(), E.states(ids))
    say(f"[gpu]   out rel-L2 {err.value:.3e}, state rel-L2 {se.value:.3e}")
    del g
    pool.close()
    assert err.value <= 1e-4 and se.value <= 1e-4
