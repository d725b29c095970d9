"""Every entry point interleaved on one pool, against the fp64 oracle.

A seeded random sequence of calls -- decode steps, windows, explicit merges,
fresh-slot assignments and flushes, each on a random subset of the slots --
drives one pool.  Every output is compared with the eager oracle, the host and
device live lengths with the closed-form schedule after every call, and the
states of all slots at the end.
"""

import numpy as np
import pytest

from workloads import CONFIGS, Workload, small_variant

pytestmark = pytest.mark.gpu

CASES = [
    # (config, overrides)
    (2, dict(H_v=4, H_k=2, d=64, L=5)),                        # GDN, fp32
    (4, dict(H_v=4, H_k=4, d=64, L=4)),                        # KDA-style, bf16 inputs
    (3, dict(H_v=4, H_k=4, d=64, L=6)),                        # GLA-style, bf16 factors
    (5, dict(H_v=4, H_k=2, d=128, L=5)),                       # GDN, bf16 state and inputs
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_mixed_calls_match_oracle(case):
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from gpu_harness import TDT, say, to_dev
    from oracle import EagerPool, RelL2, schedule

    idx, kw = CASES[case]
    P, calls = 10, 60
    cfg = small_variant(CONFIGS[idx], batch=P, num_slots=P, steps=800, replace_per_step=0, ragged_fill=False,
                        random_slots=False, name=f"mixed_{CONFIGS[idx].name}", **kw)
    wl = Workload(cfg)
    Hv, D = cfg.H_v, cfg.d
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    rng = np.random.default_rng(4242 + case)
    pool = dl.DeltaLogPool(P, Hv, cfg.H_k, D, cfg.L, cfg.decay, cfg.update, cfg.state_dtype, cfg.in_dtype,
                           max_batch=P)
    ids_all = np.arange(P, dtype=np.int32)
    pool.assign(ids_all, to_dev(wl.init_base(ids_all), st))
    E = EagerPool(ids_all, Hv, D, D, cfg.decay, cfg.update, init=wl.init_base(ids_all))
    cnt = schedule.Counters(P, cfg.L)
    bank = wl.bank_states()
    tokens = iter(wl.step_inputs(d) for d in wl.main_steps())
    say(f"[gpu] mixed calls on {cfg.describe()}")
    err, kinds = RelL2(), []

    def subset():
        n = int(rng.integers(1, P + 1))
        return np.sort(rng.choice(P, size=n, replace=False)).astype(np.int32)

    def take(ids):
        """The next token step's inputs for the entries `ids` (its rows 0..len-1)."""
        s = next(tokens)
        b = len(ids)
        return (s.q[:b], s.k[:b], s.v[:b], None if s.lam is None else s.lam[:b],
                None if s.beta is None else s.beta[:b])

    for c in range(calls):
        kind = rng.choice(["step", "step", "step", "window", "merge", "assign", "flush"], p=[.3, .15, .15, .2, .08, .08, .04])
        kinds.append(str(kind))
        if kind == "step":
            ids = subset()
            q, k, v, lam, beta = take(ids)
            out = pool.decode_step(ids, to_dev(q, it), to_dev(k, it), to_dev(v, it), to_dev(lam, torch.float32),
                                   to_dev(beta, torch.float32))
            _, o_ref = E.step(ids, q, k, v, lam, beta)
            cnt.decode(ids)
            err.add(out.cpu().numpy(), o_ref)
        elif kind == "window":
            ids = subset()
            W = int(rng.integers(1, 10))
            steps = [take(ids) for _ in range(W)]
            stack = [None if steps[0][j] is None else np.stack([s_[j] for s_ in steps]) for j in range(5)]
            q, k, v, lam, beta = stack
            out = pool.decode_window(ids, W, to_dev(q, it), to_dev(k, it), to_dev(v, it),
                                     to_dev(lam, torch.float32), to_dev(beta, torch.float32))
            for w in range(W):
                _, o_ref = E.step(ids, q[w], k[w], v[w], None if lam is None else lam[w],
                                  None if beta is None else beta[w])
                err.add(out[w].cpu().numpy(), o_ref)
            cnt.reset(ids)
        elif kind == "merge":
            ids = subset()
            pool.merge(ids)
            cnt.merge(ids)
        elif kind == "assign":
            ids = subset()
            src = rng.integers(0, len(bank), size=len(ids))
            pool.assign(ids, to_dev(bank[src], st))
            E.assign(ids, bank[src])
            cnt.reset(ids)
        else:
            pool.flush_all()
            cnt.merge(ids_all)
        torch.cuda.synchronize()
        dev_n = pool.device_log_len()
        assert np.all(pool.log_len() == cnt.n), (c, kind)
        assert np.all(dev_n == cnt.n[:, None]), (c, kind)
    for _ in range(2):                       # every slot carries rounding from a step into the final states
        q, k, v, lam, beta = take(ids_all)
        out = pool.decode_step(ids_all, to_dev(q, it), to_dev(k, it), to_dev(v, it), to_dev(lam, torch.float32),
                               to_dev(beta, torch.float32))
        _, o_ref = E.step(ids_all, q, k, v, lam, beta)
        err.add(out.cpu().numpy(), o_ref)
    pool.flush_all()
    st_e = RelL2()
    st_e.add(pool.read_base(ids_all).float().cpu().numpy(), E.states())
    tol = 2e-2 if cfg.state_dtype == "bf16" else 1e-4
    say(f"[gpu]   calls {dict((k_, kinds.count(k_)) for k_ in set(kinds))}; out rel-L2 {err.value:.3e} over "
        f"{err.count} values; state rel-L2 {st_e.value:.3e}")
    pool.close()
    assert err.value <= tol and st_e.value <= tol, (err.value, st_e.value)
    assert st_e.value > 0.0                  # the states went through the kernels' arithmetic
    assert {"step", "window", "merge", "assign"} <= set(kinds)
