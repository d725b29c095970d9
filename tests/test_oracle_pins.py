"""The oracle checked against what the pages and the mathematics fix (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle_pins as pins
from oracle import schedule
from oracle.deferred import DeferredPool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", sorted(pins.E_PINS))
def test_eager_pin(name):
    err = pins.E_PINS[name](pins.eager_step)
    assert err < 1e-12, f"{name}: {err}"


@pytest.mark.parametrize("decay,update", [("none", "plain"), ("scalar", "plain"),
                                          ("per_key", "plain"), ("scalar", "delta"),
                                          ("per_key", "delta")])
@pytest.mark.parametrize("L", [1, 2, 4, 7])
def test_deferred_equals_eager(decay, update, L):
    err = pins.pin_deferred_equals_eager(decay=decay, update=update, L=L, seed=10 + L)
    assert err < 1e-12, err


def test_deferred_L1_is_eager_every_step():
    """With M = 1 the log capacity is 0, every step merges and base == eager state."""
    rng = np.random.default_rng(3)
    F = DeferredPool(2, 2, 2, 4, 4, 1, "scalar", "delta")
    init = rng.standard_normal((2, 2, 4, 4))
    F.assign([0, 1], init)
    E = init.copy()
    for _ in range(9):
        q, k = rng.standard_normal((2, 2, 4)), rng.standard_normal((2, 2, 4))
        v = rng.standard_normal((2, 2, 4))
        lam, beta = -rng.uniform(0, 1, (2, 2)), rng.uniform(0, 1, (2, 2))
        o_f, sched = F.step([0, 1], q, k, v, lam, beta)
        E, o_e = pins.eager_step(E, q, k, v, lam, beta, "scalar", "delta")
        assert all(ph == DeferredPool.MERGE for ph, _ in sched)
        assert np.allclose(F.base, E, rtol=1e-13, atol=1e-13)
        assert np.allclose(o_f, o_e, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("L", [1, 2, 5, 16])
def test_schedule_closed_form(L):
    assert pins.pin_schedule_closed_form(L=L, seed=L) == 0


def test_schedule_formula_table():
    # a cycle is L-1 appends then one merge, counted from an empty log
    L = 4
    got = [schedule.jth_decode(0, L, j) for j in range(1, 10)]
    A, M = schedule.APPEND, schedule.MERGE
    assert got == [(A, 0), (A, 1), (A, 2), (M, 3), (A, 0), (A, 1), (A, 2), (M, 3), (A, 0)]
    # a slot that starts with 2 live entries merges on its 2nd decode
    assert [schedule.jth_decode(2, L, j)[0] for j in (1, 2, 3)] == [A, M, A]


def test_merge_on_empty_is_noop_and_flush_idempotent():
    rng = np.random.default_rng(1)
    F = DeferredPool(3, 1, 1, 3, 3, 4, "per_key", "plain")
    init = rng.standard_normal((3, 1, 3, 3))
    F.assign(range(3), init)
    F.merge([0, 1, 2])
    assert np.array_equal(F.base, init)
    x = rng.standard_normal((1, 1, 3))
    F.step([1], x, x, x, -np.ones((1, 1, 3)) * 0.2)
    S1 = F.logical_state(1)
    F.flush_all()
    assert F.n.tolist() == [0, 0, 0]
    assert np.allclose(F.base[1], S1, rtol=1e-14, atol=1e-14)
    snap = F.base.copy()
    F.flush_all()
    assert np.array_equal(F.base, snap)


def test_distinct_slot_ids_required():
    F = DeferredPool(3, 1, 1, 2, 2, 4, "none", "plain")
    x = np.ones((2, 1, 2))
    with pytest.raises(ValueError):
        F.step([1, 1], x, x, x)


def test_fpga_table2_state_bytes():
    """Eager GDN decode byte count printed by the FPGA paper (Table II)."""
    with open(os.path.join(GOLDEN, "fpga_table2_gdn_profile.json")) as f:
        g = json.load(f)
    from linear_attention_recurrent_dl_amd import traffic
    got = traffic.eager_state_bytes(H_v=g["h_v"], d_k=g["d"], d_v=g["d"], state_bytes=4)
    assert got == g["state_io_bytes"]
    # token I/O: q and k over 16 q/k heads, v and o over 32 v-heads, fp32, plus
    # four fp32 gate scalars per v-head reproduce the printed total exactly.
    tok = traffic.token_bytes(H_v=g["h_v"], H_k=16, d_k=g["d"], d_v=g["d"], in_bytes=4,
                              per_head_scalars=4)
    assert tok == g["token_io_bytes"]


# ---- the comparison machinery itself: a wrong metric or a wrong entry
#      selection would let every parity test pass without comparing anything
def test_rel_l2_metric_values():
    from oracle import RelL2
    rng = np.random.default_rng(11)
    ref = rng.standard_normal((3, 4, 5))
    m = RelL2()
    m.add(ref, ref)
    assert m.value == 0.0 and m.count == ref.size
    m = RelL2()
    m.add(2.0 * ref, ref)                       # ||2r - r|| / ||r|| = 1
    assert abs(m.value - 1.0) < 1e-15
    # streaming over pieces equals one pass over the concatenation
    x = ref + 1e-3 * rng.standard_normal(ref.shape)
    whole = RelL2()
    whole.add(x, ref)
    parts = RelL2()
    parts.add(x[:1], ref[:1])
    parts.add(x[1:], ref[1:])
    direct = np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel())
    assert abs(whole.value - direct) < 1e-15 and abs(parts.value - direct) < 1e-15
    # a NaN or an all-zero reference with a nonzero result never passes a bound
    bad = RelL2()
    bad.add(np.full(3, np.nan), np.ones(3))
    assert not (bad.value <= 1e-4)
    z = RelL2()
    z.add(np.ones(2), np.zeros(2))
    assert not (z.value <= 1e-4)
    with pytest.raises(ValueError):
        RelL2().add(np.ones(3), np.ones(4))


def test_eager_pool_steps_exactly_the_tracked_entries():
    """EagerPool follows a subset of slots: its outputs and states equal the
    eager recurrence run on exactly those batch entries, in batch order."""
    from oracle import EagerPool
    from oracle.recurrence import eager_step
    rng = np.random.default_rng(12)
    H_v, d = 2, 4
    P = 6
    init = rng.standard_normal((P, H_v, d, d))
    tracked = [4, 1, 3]
    E = EagerPool(tracked, H_v, d, d, "scalar", "delta", init=init[tracked])
    S_all = init.copy()
    for t in range(4):
        ids = rng.permutation(P)[:4]
        q, k, v = (rng.standard_normal((4, H_v, d)) for _ in range(3))
        lam = -rng.random((4, H_v))
        beta = rng.random((4, H_v))
        sel, o = E.step(ids, q, k, v, lam, beta)
        want = [j for j, s in enumerate(ids) if s in tracked]
        assert sel.tolist() == want and o.shape == (len(want), H_v, d)
        S_new, o_all = eager_step(S_all[ids], q, k, v, lam, beta, "scalar", "delta")
        S_all[ids] = S_new
        assert np.allclose(o, o_all[want], rtol=0, atol=1e-13)
    assert np.allclose(E.states(), S_all[tracked], rtol=0, atol=1e-13)
    assert np.allclose(E.states([3]), S_all[[3]], rtol=0, atol=1e-13)
