"""Degenerate inputs of the method on the GPU, against the fp64 oracle.

  beta = 0         delta rule with no correction: the state only decays
  beta = 1, |k|=1  the delta rule writes v exactly: after the step S^T k = v,
                   checked on the outputs of a step whose q equals its k
  lambda = 0       a decaying operator with no decay on this step
  lambda = -40     strong decay: the cumulative decay of older log entries
                   falls below fp32's normal range (e^-87), where the GPU
                   flushes what the oracle keeps; outputs still agree in
                   relative L2, since those entries weigh nothing
  v = 0            no new value: outputs come from the decayed state alone

Each case decodes through several merge cycles (append and merge steps,
decode steps and one window), comparing every output and the final states.
"""

import numpy as np
import pytest

from workloads import CONFIGS, Workload, small_variant

pytestmark = pytest.mark.gpu


def _edit(inp, case, rng):
    q, k, v, lam, beta = inp.q.copy(), inp.k.copy(), inp.v.copy(), inp.lam, inp.beta
    lam = None if lam is None else lam.copy()
    beta = None if beta is None else beta.copy()
    if case == "beta0":
        beta[:] = 0.0
    elif case == "beta1":
        beta[:] = 1.0
        # q = k for half of the entries' q/k heads: o = S_t^T k_t = v_t there
        q[:, ::2] = k[:, ::2]
    elif case == "lam0":
        lam[:] = 0.0
    elif case == "lam_strong":
        lam[:] = -40.0
    elif case == "v0":
        v[:] = 0.0
    return q, k, v, lam, beta


@pytest.mark.parametrize("idx", [2, 4])
@pytest.mark.parametrize("case", ["beta0", "beta1", "lam0", "lam_strong", "v0"])
def test_edge_inputs(idx, case):
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2

    base = CONFIGS[idx]
    cfg = small_variant(base, batch=3, num_slots=3, steps=30, L=4, d=64, H_v=4, H_k=2 if base.H_k < base.H_v else 4,
                        in_dtype="f32", name=f"edge_{case}_{base.name}")
    wl = Workload(cfg)
    P, Hv, D = cfg.num_slots, cfg.H_v, cfg.d
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    rng = np.random.default_rng(7)
    pool = dl.DeltaLogPool(P, Hv, cfg.H_k, D, cfg.L, cfg.decay, cfg.update, cfg.state_dtype, cfg.in_dtype,
                           max_batch=P)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, Hv, D, D, cfg.decay, cfg.update, init=wl.init_base(ids))
    say(f"[gpu] edge inputs {case}: {cfg.describe()}")
    err = RelL2()
    retrieval = []
    inputs = [_edit(wl.step_inputs(d), case, rng) for d in wl.main_steps()]
    grp = Hv // cfg.H_k
    for t, (q, k, v, lam, beta) in enumerate(inputs[:20]):
        out = pool.decode_step(ids, to_dev(q, it), to_dev(k, it), to_dev(v, it), to_dev(lam, torch.float32),
                               to_dev(beta, torch.float32)).cpu().numpy()
        _, o_ref = E.step(ids, q, k, v, lam, beta)
        err.add(out, o_ref)
        if case == "beta1":
            # v-heads whose q/k head has q = k: the output is v itself
            heads = [h for h in range(Hv) if (h // grp) % 2 == 0]
            retrieval.append(np.abs(out[:, heads] - v[:, heads]).max())
    win = inputs[20:27]
    W = len(win)
    stack = [None if win[0][j] is None else np.stack([w_[j] for w_ in win]) for j in range(5)]
    q, k, v, lam, beta = stack
    out = pool.decode_window(ids, W, to_dev(q, it), to_dev(k, it), to_dev(v, it), to_dev(lam, torch.float32),
                             to_dev(beta, torch.float32)).cpu().numpy()
    for w in range(W):
        _, o_ref = E.step(ids, q[w], k[w], v[w], None if lam is None else lam[w], None if beta is None else beta[w])
        err.add(out[w], o_ref)
    pool.flush_all()
    st_e = RelL2()
    S = pool.read_base(ids).float().cpu().numpy()
    st_e.add(S, E.states())
    say(f"[gpu]   out rel-L2 {err.value:.3e}; state rel-L2 {st_e.value:.3e}"
        + (f"; max |o - v| where q = k: {max(retrieval):.2e}" if retrieval else ""))
    pool.close()
    assert np.all(np.isfinite(S))
    assert err.value <= 1e-4 and st_e.value <= 1e-4, (err.value, st_e.value)
    if retrieval:
        assert max(retrieval) <= 1e-4


@pytest.mark.parametrize("d,tile,in_dtype,idx", [(128, 16, "f32", 2), (128, 32, "bf16", 2), (32, 32, "bf16", 1),
                                                 (16, 16, "f32", 1), (64, 32, "f32", 2), (128, 128, "f32", 2)])
def test_unwritten_log_memory_stays_out_of_outputs(d, tile, in_dtype, idx):
    """Kernels may load log entries past the live length (a whole round of the
    capacity, at small batch); whatever that memory holds must not reach the
    outputs.  The log buffers start as all-ones bytes (NaN in fp32 and bf16),
    so an entry past the live length that leaks into a sum poisons it."""
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev, tolerance
    from oracle import EagerPool, RelL2

    base = CONFIGS[idx]
    cfg = small_variant(base, batch=2, num_slots=2, steps=24, L=6, d=d, H_v=4, H_k=2 if base.H_k < base.H_v else 4,
                        in_dtype=in_dtype, name=f"stale_log_{base.name}_d{d}")
    wl = Workload(cfg)
    P, Hv, D = cfg.num_slots, cfg.H_v, cfg.d
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    pool = dl.DeltaLogPool(P, Hv, cfg.H_k, D, cfg.L, cfg.decay, cfg.update, cfg.state_dtype, cfg.in_dtype,
                           max_batch=P, value_tile=tile)
    for name in ("klog", "ulog", "lamlog"):
        pool.bufs[name].fill_(0xFF)
    ids = np.arange(P, dtype=np.int32)
    pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(ids, Hv, D, D, cfg.decay, cfg.update, init=wl.init_base(ids))
    say(f"[gpu] unwritten log memory = NaN bytes: {cfg.describe()} value_tile={pool.value_tile}")
    err = RelL2()
    finite = True
    for d_ in wl.main_steps()[:14]:
        inp = wl.step_inputs(d_)
        q, k, v, lam, beta = inp.q, inp.k, inp.v, inp.lam, inp.beta
        out = pool.decode_step(ids, to_dev(q, it), to_dev(k, it), to_dev(v, it), to_dev(lam, torch.float32),
                               to_dev(beta, torch.float32)).cpu().numpy()
        finite &= bool(np.all(np.isfinite(out)))
        _, o_ref = E.step(ids, q, k, v, lam, beta)
        err.add(out, o_ref)
    pool.flush_all()
    S = pool.read_base(ids).float().cpu().numpy()
    st_e = RelL2()
    st_e.add(S, E.states())
    say(f"[gpu]   out rel-L2 {err.value:.3e}; state rel-L2 {st_e.value:.3e}; outputs finite: {finite}")
    pool.close()
    tol = tolerance(cfg)
    assert finite and np.all(np.isfinite(S))
    assert err.value <= tol and st_e.value <= tol, (err.value, st_e.value)
