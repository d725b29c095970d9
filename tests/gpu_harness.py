"""Runs the HIP path and the fp64 oracle side by side over a workload.

Both sides read the same seeded inputs from ``workloads``; the HIP side gets
them as device tensors in the workload's dtypes, the oracle as float64.  Only
the chosen ``track`` slots are followed by the oracle (slots are independent),
so full-size workloads can be checked on a sample.
"""

from __future__ import annotations

import concurrent.futures as cf
import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import linear_attention_recurrent_dl_amd as dl
from oracle import EagerPool, RelL2, schedule
from workloads import Config, Workload

DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: Optional[np.ndarray], dtype) -> Optional[torch.Tensor]:
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def iter_inputs(wl: Workload, descs, chunk: int = 32, threads: int = 8):
    """Yield step inputs in order, generating the next chunk in the background."""
    with cf.ThreadPoolExecutor(1) as bg:
        fut = bg.submit(wl.generate, descs[:chunk], threads)
        for lo in range(0, len(descs), chunk):
            cur = fut.result()
            if lo + chunk < len(descs):
                fut = bg.submit(wl.generate, descs[lo + chunk: lo + 2 * chunk], threads)
            for inp in cur:
                yield inp


@dataclass
class Result:
    out_err: float = 0.0
    state_err: float = 0.0
    sched_mismatch: int = 0
    counter_mismatch: int = 0
    klog_mismatch: int = 0
    merges: int = 0
    appends: int = 0
    steps: int = 0
    compared_outputs: int = 0      # output values compared with the oracle
    expected_outputs: int = 0      # decoded entries of tracked slots x H_v x d
    compared_states: int = 0       # final-state values compared
    # the same errors per tracked (slot, v-head): rel-L2 of all its outputs,
    # of its final state, and the largest rel-L2 of one output vector o_t
    out_err_slot_head_max: float = 0.0
    state_err_slot_head_max: float = 0.0
    out_err_vector_max: float = 0.0
    extra: Dict[str, float] = field(default_factory=dict)


def run(cfg: Config, track: Optional[Sequence[int]] = None, steps: Optional[int] = None,
        eager: bool = False, merge_every: int = 0, check_klog: bool = True,
        value_tile: int = 0, replay_split: bool = False) -> Result:
    """Decode ``cfg`` on the GPU and in the oracle; compare outputs of tracked
    entries every step, the final state of tracked slots after a flush, the
    schedule of every entry, and the device counters of every slot."""
    wl = Workload(cfg)
    P, Hv, Hk, D = cfg.num_slots, cfg.H_v, cfg.H_k, cfg.d
    track = list(range(P)) if track is None else sorted(int(s) for s in track)
    L = 1 if eager else cfg.L
    say(f"[gpu] {cfg.describe()} eager={eager} track={len(track)} slots value_tile={value_tile} "
        f"replay_split={replay_split}")
    pool = dl.DeltaLogPool(P, Hv, Hk, D, L, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, max_batch=cfg.batch, value_tile=value_tile,
                           replay_split=replay_split)
    st, it = TDT[cfg.state_dtype], TDT[cfg.in_dtype]
    # initial states: every slot gets its seeded base (chunks of max_batch)
    for lo in range(0, P, cfg.batch):
        ids = np.arange(lo, min(P, lo + cfg.batch), dtype=np.int32)
        pool.assign(ids, to_dev(wl.init_base(ids), st))
    E = EagerPool(track, Hv, D, D, cfg.decay, cfg.update, init=wl.init_base(track))
    cnt = schedule.Counters(P, L)
    bank = to_dev(wl.bank_states(), st) if cfg.replace_per_step else None
    bank_np = wl.bank_states() if cfg.replace_per_step else None

    res = Result()
    out_e = RelL2()
    sh_num = np.zeros((len(track), Hv))            # per (tracked slot, v-head) squared error / norm
    sh_den = np.zeros((len(track), Hv))
    trow = {s: i for i, s in enumerate(track)}
    tracked = set(track)
    klog_written: Dict[int, Dict[int, np.ndarray]] = {s: {} for s in track}
    descs = wl.plan(steps)
    step_fn = pool.eager_step if eager else pool.decode_step
    for si, inp in enumerate(iter_inputs(wl, descs)):
        if len(inp.replace_ids):
            pool.assign(inp.replace_ids, bank[torch.from_numpy(inp.replace_bank.astype(np.int64)).to(DEV)].contiguous())
            E.assign(inp.replace_ids, bank_np[inp.replace_bank])
            cnt.reset(inp.replace_ids)
            for s in inp.replace_ids:
                if int(s) in tracked:
                    klog_written[int(s)] = {}
        ids = inp.slot_ids
        merge, index = pool.schedule(ids)
        want = cnt.decode(ids)
        res.sched_mismatch += int(sum(int(m) != int(ph == schedule.MERGE) or int(ix) != int(wix)
                                      for m, ix, (ph, wix) in zip(merge, index, want)))
        res.merges += int(merge.sum())
        res.appends += int(len(ids) - merge.sum())
        q, k, v = to_dev(inp.q, it), to_dev(inp.k, it), to_dev(inp.v, it)
        lam = to_dev(inp.lam, torch.float32)
        beta = to_dev(inp.beta, torch.float32)
        out = step_fn(ids, q, k, v, lam, beta)
        sel, o_ref = E.step(ids, inp.q, inp.k, inp.v, inp.lam, inp.beta)
        res.expected_outputs += sum(int(s) in tracked for s in ids) * Hv * D
        if len(sel):
            o_gpu = out[torch.from_numpy(sel).to(DEV)].cpu().numpy()
            out_e.add(o_gpu, o_ref)
            d2 = np.sum((o_gpu.astype(np.float64) - o_ref) ** 2, axis=-1)      # [n, H_v]
            r2 = np.sum(o_ref ** 2, axis=-1)
            rows = [trow[int(ids[e])] for e in sel]
            np.add.at(sh_num, rows, d2)
            np.add.at(sh_den, rows, r2)
            nz = r2 > 0
            if np.any(nz):
                res.out_err_vector_max = max(res.out_err_vector_max, float(np.sqrt(np.max(d2[nz] / r2[nz]))))
            if check_klog and not eager:
                for e in sel:
                    s = int(ids[e])
                    if merge[e]:
                        klog_written[s] = {}
                    else:
                        klog_written[s][int(index[e])] = inp.k[e]
        if merge_every and (si + 1) % merge_every == 0 and not eager:
            ms = np.array(track[: max(1, len(track) // 2)], dtype=np.int32)
            for lo in range(0, len(ms), cfg.batch):
                pool.merge(ms[lo: lo + cfg.batch])
            cnt.merge(ms)
            for s in ms:
                klog_written[int(s)] = {}
        res.steps += 1
    torch.cuda.synchronize()
    # bookkeeping: device counters (every head of every slot) and host mirror
    dev_n = pool.device_log_len()
    res.counter_mismatch = int(np.sum(dev_n != cnt.n[:, None])) + int(np.sum(pool.log_len() != cnt.n))
    # lossless key-factor copies of the live log of tracked slots
    if check_klog and not eager and L > 1:
        kl = pool.bufs["klog"][: pool.sizes[1]].view(it).view(P, Hk, L - 1, D).cpu().float().numpy()
        for s in track:
            for i, kin in klog_written[s].items():
                res.klog_mismatch += int(np.sum(kl[s, :, i] != kin))
    pool.flush_all()
    torch.cuda.synchronize()
    res.counter_mismatch += int(np.sum(pool.device_log_len() != 0))
    S_gpu = pool.read_base(track).float().cpu().numpy()
    st_e = RelL2()
    S_ref = E.states()
    st_e.add(S_gpu, S_ref)
    res.out_err, res.state_err = out_e.value, st_e.value
    seen = sh_den > 0
    if np.any(seen):
        res.out_err_slot_head_max = float(np.sqrt(np.max(sh_num[seen] / sh_den[seen])))
    s_num = np.sum((S_gpu.astype(np.float64) - S_ref) ** 2, axis=(2, 3))
    s_den = np.sum(S_ref ** 2, axis=(2, 3))
    if np.any(s_den > 0):
        res.state_err_slot_head_max = float(np.sqrt(np.max(s_num[s_den > 0] / s_den[s_den > 0])))
    res.compared_outputs, res.compared_states = out_e.count, st_e.count
    say(f"[gpu]   per (slot, head) max: out rel-L2 {res.out_err_slot_head_max:.3e}  state rel-L2 "
        f"{res.state_err_slot_head_max:.3e}; largest single-output rel-L2 {res.out_err_vector_max:.3e}")
    say(f"[gpu]   out rel-L2 {res.out_err:.3e}  state rel-L2 {res.state_err:.3e}  "
        f"merges {res.merges} appends {res.appends}  sched-mismatch {res.sched_mismatch}  "
        f"counter-mismatch {res.counter_mismatch}  klog-mismatch {res.klog_mismatch}")
    pool.close()
    return res


def tolerance(cfg: Config) -> float:
    """rel-L2 bound on outputs and states: 1e-4 for fp32 state, 2e-2 for bf16 state."""
    return 2e-2 if cfg.state_dtype == "bf16" else 1e-4
