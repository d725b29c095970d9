"""dl_decode_step_noalloc, the decode entry point that allocates nothing,
against dl_decode_step on the same inputs.

Two pools of the same split-replay descriptor start from the same states: one
with its own coefficient buffer, decoded by dl_decode_step, the other created
without it, decoded by dl_decode_step_noalloc (the library's static scratch
holds the coefficients).  Every call's outputs and the final states must be
identical (the kernels and their arithmetic are the same), and within the
oracle's tolerance.  Two calls in a row, the second with a smaller batch, then
more steps through merges; one descriptor needs several launches per call
because the static scratch holds fewer slots than a call carries.
"""

import numpy as np
import pytest

import linear_attention_recurrent_dl_amd as dl
from linear_attention_recurrent_dl_amd import _native as N
from workloads import CONFIGS, Workload, small_variant


def test_noalloc_refuses_a_pool_whose_slot_exceeds_the_scratch():
    # host-only pools validate exactly as device pools do
    big = dl.DeltaLogPool(2, 16384, 16384, 16, 64, "scalar", "delta", max_batch=2, device=None,
                          replay_split=True)
    with pytest.raises(dl.DeltaLogError) as ei:
        big.decode_step_noalloc([0])
    assert ei.value.code == N.DL_ERR_UNSUPPORTED and "static scratch" in str(ei.value)
    assert np.all(big.log_len() == 0)
    ok = dl.DeltaLogPool(4, 8, 4, 16, 4, "scalar", "delta", max_batch=4, device=None, replay_split=True)
    ok.decode_step_noalloc([0, 2])
    assert list(ok.log_len()) == [1, 0, 1, 0]
    big.close()
    ok.close()


CASES = [
    # (base config, overrides): GDN-style and KDA-style split pools; the last
    # one needs 4096 floats per slot, so a 300-slot call is two launches
    (2, dict(batch=12, num_slots=12, steps=9, H_v=8, H_k=4, L=4)),
    (4, dict(batch=10, num_slots=10, steps=7, H_v=4, H_k=4, L=6)),
    (2, dict(batch=300, num_slots=300, steps=3, H_v=32, H_k=16, d=32, L=64)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("idx,kw", CASES, ids=["gdn", "kda", "gdn_two_launches"])
def test_noalloc_matches_decode_step(idx, kw):
    import torch

    from gpu_harness import TDT, say, to_dev, tolerance
    from oracle import EagerPool, RelL2

    cfg = small_variant(CONFIGS[idx], name=f"noalloc_{CONFIGS[idx].name}", random_slots=False, replace_per_step=0,
                        ragged_fill=False, **kw)
    say(f"[gpu] no-alloc entry point vs dl_decode_step: {cfg.describe()}")
    wl = Workload(cfg)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    P = cfg.num_slots
    mk = dict(max_batch=cfg.batch, replay_split=True)
    ref = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype, cfg.in_dtype,
                          **mk)
    na = dl.DeltaLogPool(P, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update, cfg.state_dtype, cfg.in_dtype,
                         coef_buffer=False, **mk)
    assert na.bufs["coef"].numel() == 16 and ref.sizes[5] > 0
    ids = np.arange(P, dtype=np.int32)
    init = wl.init_base(ids)
    ref.assign(ids, to_dev(init, st))
    na.assign(ids, to_dev(init, st))
    E = EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=init)
    err = RelL2()
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    s0 = steps[0]
    with pytest.raises(dl.DeltaLogError) as ei:    # no coefficient buffer: only the no-alloc entry point decodes it
        na.decode_step(s0.slot_ids, to_dev(s0.q, it), to_dev(s0.k, it), to_dev(s0.v, it),
                       None if s0.lam is None else to_dev(s0.lam, torch.float32),
                       None if s0.beta is None else to_dev(s0.beta, torch.float32))
    assert ei.value.code == N.DL_ERR_INVALID_ARG and np.all(na.log_len() == 0)
    for t, s in enumerate(steps):
        # the second call of the run decodes fewer slots than the first
        sel = np.arange(P) if t != 1 else np.arange(0, P, 3)
        sid = s.slot_ids[sel]
        args = (to_dev(s.q[sel], it), to_dev(s.k[sel], it), to_dev(s.v[sel], it),
                None if s.lam is None else to_dev(s.lam[sel], torch.float32),
                None if s.beta is None else to_dev(s.beta[sel], torch.float32))
        o_ref = ref.decode_step(sid, *args)
        o_na = na.decode_step_noalloc(sid, *args)
        _, o_e = E.step(sid, s.q[sel], s.k[sel], s.v[sel], None if s.lam is None else s.lam[sel],
                        None if s.beta is None else s.beta[sel])
        torch.cuda.synchronize()
        a, b = o_ref.cpu().numpy(), o_na.cpu().numpy()
        say(f"[gpu]   call {t}: {len(sid)} slots, max |diff| {np.abs(a - b).max():.3e}")
        assert np.array_equal(a, b), f"call {t}: outputs differ"
        err.add(b, o_e)
    assert np.array_equal(ref.log_len(), na.log_len())
    assert np.array_equal(ref.device_log_len(), na.device_log_len())
    ref.flush_all()
    na.flush_all()
    Sr = ref.read_base(ids).float().cpu().numpy()
    Sn = na.read_base(ids).float().cpu().numpy()
    st_e = RelL2()
    st_e.add(Sn, E.states())
    say(f"[gpu]   out rel-L2 {err.value:.3e}, state rel-L2 {st_e.value:.3e}")
    ref.close()
    na.close()
    assert np.array_equal(Sr, Sn)
    tol = tolerance(cfg)
    assert err.value <= tol and st_e.value <= tol
