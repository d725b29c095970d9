"""The window entry point (W consecutive steps of the same slots in one launch,
state held in registers) against the fp64 oracle.

Each case decodes a few ordinary steps first, so that the window starts from
live logs of several lengths (ragged fills, full logs about to merge), then
runs one window, then ordinary steps again, then flushes.  Every output of
every step and the final states are compared with the eager oracle run step by
step; live lengths must be zero for the windowed slots and follow the closed-form
schedule for every other call.
"""

import numpy as np
import pytest

from workloads import CONFIGS, Workload, small_variant

pytestmark = pytest.mark.gpu


def _stack(inputs, name):
    xs = [getattr(s, name) for s in inputs]
    return None if xs[0] is None else np.stack(xs)


def run_window_case(cfg, W, value_tile=0, pre=None, post=3, window_slots=None, track=None):
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2, schedule

    wl = Workload(cfg)
    P, Hv, D = cfg.num_slots, cfg.H_v, cfg.d
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    pool = dl.DeltaLogPool(P, Hv, cfg.H_k, D, cfg.L, cfg.decay, cfg.update, cfg.state_dtype, cfg.in_dtype,
                           max_batch=max(cfg.batch, P), value_tile=value_tile)
    ids_all = np.arange(P, dtype=np.int32)
    pool.assign(ids_all, to_dev(wl.init_base(ids_all), st))
    tracked = ids_all if track is None else np.asarray(sorted(track), dtype=np.int32)
    E = EagerPool(tracked, Hv, D, D, cfg.decay, cfg.update, init=wl.init_base(tracked))
    cnt = schedule.Counters(P, cfg.L)
    descs = wl.plan()
    pre = len(wl.fill_steps()) + (cfg.L // 2 if pre is None else pre)
    assert pre + W + post <= len(descs)
    say(f"[gpu] window W={W} after {pre} steps: {cfg.describe()} value_tile={pool.value_tile}")
    out_e, n_out = RelL2(), 0

    def step(inp):
        nonlocal n_out
        out = pool.decode_step(inp.slot_ids, to_dev(inp.q, it), to_dev(inp.k, it), to_dev(inp.v, it),
                               to_dev(inp.lam, torch.float32), to_dev(inp.beta, torch.float32))
        sel, o_ref = E.step(inp.slot_ids, inp.q, inp.k, inp.v, inp.lam, inp.beta)
        cnt.decode(inp.slot_ids)
        if len(sel):
            out_e.add(out.cpu().numpy()[sel], o_ref)
        n_out += out.numel()

    inputs = [wl.step_inputs(d) for d in descs[: pre + W + post]]
    for inp in inputs[:pre]:
        step(inp)
    n_before = cnt.n.copy()
    # the window: the slots of its first step, the token inputs of W steps
    win = inputs[pre: pre + W]
    ids = win[0].slot_ids if window_slots is None else np.asarray(window_slots, dtype=np.int32)
    B = len(ids)
    q, k, v = (_stack(win, x)[:, :B] for x in ("q", "k", "v"))
    lam, beta = _stack(win, "lam"), _stack(win, "beta")
    lam = None if lam is None else lam[:, :B]
    beta = None if beta is None else beta[:, :B]
    out = pool.decode_window(ids, W, to_dev(q, it), to_dev(k, it), to_dev(v, it), to_dev(lam, torch.float32),
                             to_dev(beta, torch.float32))
    win_e = RelL2()
    for w in range(W):
        sel, o_ref = E.step(ids, q[w], k[w], v[w], None if lam is None else lam[w], None if beta is None else beta[w])
        win_e.add(out[w].cpu().numpy()[sel], o_ref)
    cnt.reset(ids)
    torch.cuda.synchronize()
    dev_n = pool.device_log_len()
    counter_mismatch = int(np.sum(dev_n != cnt.n[:, None])) + int(np.sum(pool.log_len() != cnt.n))
    for inp in inputs[pre + W:]:
        step(inp)
    pool.flush_all()
    torch.cuda.synchronize()
    st_e = RelL2()
    st_e.add(pool.read_base(tracked).float().cpu().numpy(), E.states())
    counter_mismatch += int(np.sum(pool.device_log_len() != 0))
    say(f"[gpu]   window out rel-L2 {win_e.value:.3e} over {win_e.count} values; steps {out_e.value:.3e}; "
        f"state {st_e.value:.3e}; live lengths before {sorted(set(n_before[ids].tolist()))}; "
        f"counter mismatch {counter_mismatch}")
    pool.close()
    tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
    assert win_e.count == W * int(np.isin(ids, tracked).sum()) * Hv * D
    assert win_e.value <= tol and out_e.value <= tol and st_e.value <= tol, (win_e.value, out_e.value, st_e.value)
    assert counter_mismatch == 0
    return n_before[ids]


def _small(idx, **kw):
    base = CONFIGS[idx]
    ch = dict(batch=3, H_v=4, H_k=2 if base.H_k < base.H_v else 4, L=5, steps=40, replace_per_step=0,
              name=f"window_{base.name}")
    if base.random_slots:
        ch.update(num_slots=7)
    ch.update(kw)
    return small_variant(base, **ch)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("W", [1, 6, 17])
def test_window_matches_oracle(idx, W):
    run_window_case(_small(idx), W)


@pytest.mark.parametrize("idx,value_tile", [(2, 32), (2, 16), (4, 32), (3, 32), (5, 64)])
def test_window_value_tiles(idx, value_tile):
    run_window_case(_small(idx), 9, value_tile=value_tile)


def test_window_from_full_logs():
    """Every windowed slot holds L - 1 entries: the window materializes full logs."""
    cfg = _small(2, L=4)
    n0 = run_window_case(cfg, 5, pre=3)
    assert set(n0.tolist()) == {3}


def test_window_from_ragged_logs():
    """Serving-pool shape: random slots, ragged initial fills, a window over a
    subset of the pool while other slots keep their logs."""
    cfg = _small(5, num_slots=9, batch=4, L=6, ragged_fill=True)
    n0 = run_window_case(cfg, 7, pre=2, window_slots=[8, 0, 5, 3])
    assert len(set(n0.tolist())) > 1


def test_window_long_and_chunked_launch():
    """W = 300 and the largest window, W = 4096; and 520 slots: more entries
    than one launch carries."""
    run_window_case(_small(1, L=8, steps=320), 300, pre=2, post=2)
    run_window_case(_small(1, L=8, steps=4104), 4096, pre=2, post=2)
    run_window_case(_small(1, batch=520, num_slots=520, H_v=2, H_k=2, steps=12), 5, pre=2, post=2)


def test_window_headline_shape():
    """GDN, 32 v-heads / 16 q/k heads, d = 128, fp32, batch 1, L = 16: one window of 16 steps."""
    cfg = small_variant(CONFIGS[2], steps=48, name="window_gdn_b1_h32_d128")
    run_window_case(cfg, 16, pre=7)


@pytest.mark.parametrize("idx", [2, 4, 5])
def test_window_graph_replay(idx):
    """A window launch captured in a HIP graph and replayed three times, with
    eager device work between replays: each replay applies the same W steps to
    the state the previous one left, and every output matches the oracle."""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    cfg = _small(idx, ragged_fill=False)
    wl = Workload(cfg)
    P, Hv, D, W = cfg.num_slots, cfg.H_v, cfg.d, 7
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    pool = dl.DeltaLogPool(P, Hv, cfg.H_k, D, cfg.L, cfg.decay, cfg.update, cfg.state_dtype, cfg.in_dtype,
                           max_batch=P)
    ids_all = np.arange(P, dtype=np.int32)
    pool.assign(ids_all, to_dev(wl.init_base(ids_all), st))
    E = EagerPool(ids_all, Hv, D, D, cfg.decay, cfg.update, init=wl.init_base(ids_all))
    win = [wl.step_inputs(d) for d in wl.main_steps(W)]
    ids = win[0].slot_ids
    q, k, v = (_stack(win, x) for x in ("q", "k", "v"))
    lam, beta = _stack(win, "lam"), _stack(win, "beta")
    dq, dk, dv = to_dev(q, it), to_dev(k, it), to_dev(v, it)
    dlam, dbeta = to_dev(lam, torch.float32), to_dev(beta, torch.float32)
    out = torch.empty((W, len(ids), Hv, D), dtype=torch.float32, device="cuda")
    say(f"[gpu] window graph replay {cfg.describe()} W={W}")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pool.decode_window(ids, W, dq, dk, dv, dlam, dbeta, out)
    scratch = torch.randn(1 << 20, device="cuda")
    tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        err = RelL2()
        for w in range(W):
            _, o_ref = E.step(ids, q[w], k[w], v[w], None if lam is None else lam[w],
                              None if beta is None else beta[w])
            err.add(out[w].cpu().numpy(), o_ref)
        scratch.mul_(0.5).add_(1.0)
        torch.cuda.synchronize()
        say(f"[gpu]   replay {rep}: out rel-L2 {err.value:.3e}")
        assert err.value <= tol
        assert np.all(pool.device_log_len()[ids] == 0)
    st_e = RelL2()
    st_e.add(pool.read_base(ids_all).float().cpu().numpy(), E.states())
    assert st_e.value <= tol
    pool.close()


def test_window_full_size_sampled():
    """The benchmark's batch window: GDN, batch 128, 32 v-heads, d = 128, fp32,
    default value tiles, W = 64, after a few steps of every slot; three slots
    followed by the oracle."""
    from workloads import headline_gdn
    cfg = headline_gdn(128, steps=80)
    run_window_case(cfg, 64, pre=5, post=3, track=[0, 77, 127])


@pytest.mark.parametrize("idx", [2, 4])
def test_window_on_eager_pool(idx):
    """Merge interval 1 (no log; steps run the eager kernel): the window
    materializes nothing and carries the state through its steps."""
    run_window_case(_small(idx, L=1), 6, pre=3)
