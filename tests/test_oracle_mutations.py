"""Plant plausible mistakes in copies of the oracle and check that a pin catches each.

The mutants live here, on the CPU; the oracle itself is untouched.
"""

import numpy as np
import pytest

import oracle_pins as pins
from oracle.deferred import DeferredPool
from oracle.recurrence import decay_factors, expand_heads


def mutant_eager_step(flag):
    def step(S, q, a_or_k, b_or_v, lam, beta, decay, update):
        S = np.asarray(S, dtype=np.float64)
        N, H_v, d_k, d_v = S.shape
        if flag == "tiled_heads":
            qv = np.tile(np.asarray(q, dtype=np.float64), (1, H_v // q.shape[1], 1))
            av = np.tile(np.asarray(a_or_k, dtype=np.float64), (1, H_v // q.shape[1], 1))
        else:
            qv, av = expand_heads(q, H_v), expand_heads(a_or_k, H_v)
        if flag == "neg_exp" and lam is not None:
            lam = -np.asarray(lam)
        g = decay_factors(lam, N, H_v, d_k, decay)
        P = g[..., None, :] * S if flag == "decay_columns" else g[..., :, None] * S
        if update == "delta":
            src = S if flag == "undecayed_correction" else P
            PTk = np.einsum("nhrc,nhr->nhc", src, av)
            bt = np.asarray(beta, dtype=np.float64)[..., None]
            if flag == "drop_beta":
                bt = np.ones_like(bt)
            if flag == "sign_flip":
                b = bt * (b_or_v + PTk)
            else:
                b = bt * (b_or_v - PTk)
        else:
            b = np.asarray(b_or_v, dtype=np.float64)
        if flag == "outer_transposed":
            S_new = P + b[..., :, None] * av[..., None, :]
        else:
            S_new = P + av[..., :, None] * b[..., None, :]
        if flag == "output_from_previous":
            o = np.einsum("nhrc,nhr->nhc", P, qv)
        elif flag == "output_untransposed":
            o = np.einsum("nhrc,nhc->nhr", S_new, qv)
        else:
            o = np.einsum("nhrc,nhr->nhc", S_new, qv)
        return S_new, o
    return step


E_FLAGS = ["tiled_heads", "neg_exp", "decay_columns", "undecayed_correction", "drop_beta",
           "sign_flip", "outer_transposed", "output_from_previous", "output_untransposed"]


def _caught(run) -> bool:
    try:
        return run() > 1e-6
    except Exception:
        return True


@pytest.mark.parametrize("flag", E_FLAGS)
def test_eager_mutant_is_caught(flag):
    step = mutant_eager_step(flag)
    caught = [name for name, pin in pins.E_PINS.items() if _caught(lambda: pin(step))]
    assert caught, f"no pin catches mutant {flag}"


def test_unmutated_copy_passes_every_pin():
    step = mutant_eager_step("none")
    for name, pin in pins.E_PINS.items():
        assert pin(step) < 1e-12, name


class MutantDeferred(DeferredPool):
    flag = None

    def step(self, slots, q, a_or_k, b_or_v, lam=None, beta=None):
        slots = np.asarray(slots, dtype=np.int64)
        qv, av = expand_heads(q, self.H_v), expand_heads(a_or_k, self.H_v)
        bv = np.asarray(b_or_v, dtype=np.float64)
        out = np.zeros((len(slots), self.H_v, self.d_v))
        sched = []
        for e, s in enumerate(slots):
            lam_e = self._lam_vec(None if lam is None else lam[e])
            lprime = self.lbar[s] + lam_e
            a = av[e]
            if self.update == "delta":
                b = np.asarray(beta[e])[:, None] * (bv[e] - self._replay_transpose(s, lprime, a))
            else:
                b = bv[e]
            out[e] = self._replay_transpose(s, lprime, qv[e]) + np.sum(a * qv[e], axis=-1)[:, None] * b
            n = int(self.n[s])
            merge_at = self.C - 1 if self.flag == "early_merge" else self.C
            if n >= merge_at:
                S = np.exp(lprime)[:, :, None] * self.base[s]
                for i in range(n):
                    w = np.exp(self.Lam[s, :, i] - lprime) if self.flag == "weight_inverted" \
                        else np.exp(lprime - self.Lam[s, :, i])
                    S = S + (w * self.K[s, :, i])[:, :, None] * self.U[s, :, i][:, None, :]
                if self.flag != "merge_drops_token":
                    S = S + a[:, :, None] * b[:, None, :]
                self.base[s] = S
                self.lbar[s] = 0.0
                self.n[s] = 0
                sched.append((self.MERGE, n))
            else:
                self.K[s, :, n] = a
                self.U[s, :, n] = b
                self.Lam[s, :, n] = self.lbar[s] if self.flag == "snapshot_before_decay" else lprime
                self.lbar[s] = lprime
                self.n[s] = n + 1
                sched.append((self.APPEND, n))
        return out, sched


F_FLAGS = ["early_merge", "weight_inverted", "merge_drops_token", "snapshot_before_decay"]


@pytest.mark.parametrize("flag", F_FLAGS)
def test_deferred_mutant_is_caught(flag):
    cls = type("M_" + flag, (MutantDeferred,), {"flag": flag})
    runs = [
        lambda: pins.pin_deferred_equals_eager(pool_cls=cls, decay="per_key", update="delta", L=4),
        lambda: pins.pin_deferred_equals_eager(pool_cls=cls, decay="scalar", update="plain", L=3),
        lambda: float(pins.pin_schedule_closed_form(pool_cls=cls, L=5)),
    ]
    assert any(_caught(r) for r in runs), f"no pin catches deferred mutant {flag}"


def test_unmutated_deferred_copy_passes():
    cls = type("M_none", (MutantDeferred,), {"flag": "none"})
    assert pins.pin_deferred_equals_eager(pool_cls=cls, decay="per_key", update="delta", L=4) < 1e-12
    assert pins.pin_schedule_closed_form(pool_cls=cls, L=5) == 0
