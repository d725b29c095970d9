"""Host logic of bench.py (no GPU): measurement windows, workload tags, the
one-GPU contract."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("R,L,at_least,want", [(1, 16, 64, 64), (3, 16, 64, 96), (21, 32, 128, 672), (5, 16, 16, 80),
                                               (1, 8, 1, 8)])
def test_cycle_steps_are_whole_cycles_of_every_pool(R, L, at_least, want):
    s = bench.cycle_steps(R, L, at_least)
    assert s == want
    assert s % (R * L) == 0 and s >= at_least


def test_workload_tags():
    from workloads import CONFIGS
    assert bench.extra_cfg("2") == CONFIGS[2]
    g = bench.extra_cfg("g128")
    assert (g.batch, g.num_slots, g.H_v, g.H_k, g.d, g.state_dtype) == (128, 128, 32, 16, 128, "f32")
    k = bench.extra_cfg("k256")
    base4 = CONFIGS[4]
    assert (k.batch, k.num_slots, k.H_v, k.H_k, k.d, k.decay, k.update, k.L) == (
        256, 256, base4.H_v, base4.H_k, base4.d, base4.decay, base4.update, base4.L)
    share = bench.extra_cfg("5tp8")
    base = CONFIGS[5]
    # one GPU's share under 8-way head sharding: every slot, a slice of the heads
    assert (share.num_slots, share.batch, share.H_v, share.H_k) == (base.num_slots, base.batch, 4, 2)
    assert (share.decay, share.update, share.state_dtype, share.L) == (base.decay, base.update, base.state_dtype,
                                                                       base.L)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["requested_gpus"] == 2 and "one GPU" in line["error"]
    assert "--gpus 1" in r.stderr
