"""The numerical campaign of the DeltaLog paper's kernel evaluation, repeated
against the fp64 oracle: 128-token rollouts at batch 64, 128 and 256 for the
GDN, KDA-style and GLA/RWKV6-style operators, each with its workload's merge
interval, dtypes and input distributions.

The paper reports the largest output and state relative errors of such
rollouts against dense references.  Here the bound of the fp32-state
workloads (rel-L2 <= 1e-4) is asserted pooled over the sampled slots, and
again for every sampled (slot, v-head) on its own -- all of its 128 outputs,
and its final state -- so that an error confined to one slot-head or one
stretch of steps cannot hide in the pooled figure.  The largest rel-L2 of a
single output vector is reported alongside (line "[numerics]").
"""

import pytest

from workloads import CONFIGS, at_batch, headline_gdn

pytestmark = pytest.mark.gpu

STEPS = 128


def _config(op, B):
    if op == "gdn":
        return headline_gdn(B, steps=STEPS)
    return at_batch(CONFIGS[4 if op == "kda" else 3], B, steps=STEPS)


@pytest.mark.parametrize("B", [64, 128, 256])
@pytest.mark.parametrize("op", ["gdn", "kda", "gla"])
def test_rollout_128_tokens(op, B):
    from gpu_harness import run, say, tolerance
    cfg = _config(op, B)
    track = [0, B // 3, (2 * B) // 3 + 1, B - 1]
    res = run(cfg, track=track)
    tol = tolerance(cfg)
    say(f"[numerics] {op} B={B} L={cfg.L} d={cfg.d} state={cfg.state_dtype} in={cfg.in_dtype}: "
        f"out pooled {res.out_err:.3e} max(slot,head) {res.out_err_slot_head_max:.3e} "
        f"max(vector) {res.out_err_vector_max:.3e} | state pooled {res.state_err:.3e} "
        f"max(slot,head) {res.state_err_slot_head_max:.3e}")
    assert res.steps == STEPS and res.compared_outputs == res.expected_outputs > 0
    assert res.sched_mismatch == 0 and res.counter_mismatch == 0 and res.klog_mismatch == 0
    assert res.out_err <= tol and res.state_err <= tol
    assert res.out_err_slot_head_max <= tol, f"a (slot, head) has output rel-L2 {res.out_err_slot_head_max:.3e}"
    assert res.state_err_slot_head_max <= tol, f"a (slot, head) has state rel-L2 {res.state_err_slot_head_max:.3e}"
