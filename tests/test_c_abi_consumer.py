"""The C ABI from plain C: a gcc-built consumer (tests/c_abi/dl_c_consumer.c)
that allocates with hipMalloc and drives the library with no Python in the
loop.  The host-only mode runs here; the GPU mode is compared with the fp64
oracle on the GPU."""

import os
import subprocess

import numpy as np
import pytest

from oracle import EagerPool, RelL2, schedule
from workloads import CONFIGS, Workload, small_variant

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "dl_c_consumer")


def _binary() -> str:
    if not os.path.exists(BIN):
        raise RuntimeError(f"{BIN} is missing; run the build step (__graft_entry__.build() or "
                           "python tests/c_abi/build_consumer.py)")
    return BIN


def test_c_consumer_host_only_schedule():
    """Host-only pool from C: live lengths after each call follow the closed-form schedule."""
    r = subprocess.run([_binary(), "--dry"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    rows = [list(map(int, line.split())) for line in r.stdout.split("\n") if line.strip()]
    cnt = schedule.Counters(3, 4)
    want = []
    for t in range(6):
        if t == 2:
            cnt.merge([2])
        cnt.decode([0, 1, 2] if t % 2 == 0 else [2, 0])
        want.append(cnt.n.tolist())
    want.append(cnt.n.tolist())             # the refused duplicate call changes nothing
    assert rows == want


def _write(dirpath, cfg, value_tile=0, split=0, window=0):
    wl = Workload(cfg)
    ids_all = np.arange(cfg.num_slots, dtype=np.int32)
    init = wl.init_base(ids_all).astype(np.float32)
    steps = [wl.step_inputs(d) for d in wl.main_steps()]
    decay = {"none": 0, "scalar": 1, "per_key": 2}[cfg.decay]
    update = {"plain": 0, "delta": 1}[cfg.update]
    with open(os.path.join(dirpath, "desc.txt"), "w") as f:
        f.write(f"{cfg.num_slots} {cfg.batch} {cfg.H_v} {cfg.H_k} {cfg.d} {cfg.L} {decay} {update} "
                f"{len(steps)} {value_tile} {split} {window}\n")
    init.tofile(os.path.join(dirpath, "init.bin"))
    np.stack([s.slot_ids for s in steps]).astype(np.int32).tofile(os.path.join(dirpath, "ids.bin"))
    for name in ("q", "k", "v"):
        np.stack([getattr(s, name) for s in steps]).astype(np.float32).tofile(os.path.join(dirpath, name + ".bin"))
    if cfg.decay != "none":
        np.stack([s.lam for s in steps]).astype(np.float32).tofile(os.path.join(dirpath, "lam.bin"))
    if cfg.update == "delta":
        np.stack([s.beta for s in steps]).astype(np.float32).tofile(os.path.join(dirpath, "beta.bin"))
    return init, steps


@pytest.mark.gpu
@pytest.mark.parametrize("base_idx,value_tile,split,window", [(2, 32, 0, 0), (2, 32, 1, 0), (4, 64, 0, 0), (1, 0, 0, 0),
                                                              (2, 32, 0, 9), (4, 64, 0, 23)])
def test_c_consumer_matches_oracle(tmp_path, base_idx, value_tile, split, window):
    base = CONFIGS[base_idx]
    cfg = small_variant(base, batch=3, steps=23, L=5, H_v=4, H_k=2 if base.H_k < base.H_v else 4,
                        in_dtype="f32", state_dtype="f32", name=f"c_abi_{base.name}")
    init, steps = _write(str(tmp_path), cfg, value_tile, split, window)
    print(f"[gpu] C consumer on {cfg.describe()} value_tile={value_tile} split={split} window={window}", flush=True)
    r = subprocess.run([_binary(), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    B, Hv, D, P = cfg.batch, cfg.H_v, cfg.d, cfg.num_slots
    out = np.fromfile(os.path.join(tmp_path, "out.bin"), dtype=np.float32).reshape(len(steps), B, Hv, D)
    state = np.fromfile(os.path.join(tmp_path, "state.bin"), dtype=np.float32).reshape(P, Hv, D, D)
    E = EagerPool(range(P), Hv, D, D, cfg.decay, cfg.update, init=init)
    cnt = schedule.Counters(P, cfg.L)
    err = RelL2()
    for t, s in enumerate(steps):
        sel, o_ref = E.step(s.slot_ids, s.q, s.k, s.v, s.lam, s.beta)
        if t < len(steps) - window:
            cnt.decode(s.slot_ids)
        err.add(out[t][sel], o_ref)
    if window:
        cnt.reset(steps[-1].slot_ids)          # a window leaves the log empty
    st = RelL2()
    st.add(state, E.states())
    assert err.count == len(steps) * B * Hv * D
    assert err.value <= 1e-4 and st.value <= 1e-4, (err.value, st.value)
    lines = open(os.path.join(tmp_path, "loglen.txt")).read().split("\n")
    assert list(map(int, lines[0].split())) == cnt.n.tolist()
    assert int(lines[1]) == 0                  # every device counter empty after the flush
