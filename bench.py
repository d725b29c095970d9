#!/usr/bin/env python3
"""DeltaLog decode-step benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload N] [--no-extra] [--no-cpu]
    python bench.py --sweep merge|state

A step is one decode of the workload's batch (for the serving pool: its fresh
slot assignments, then the decode).  The headline workload is the 32-v-head
d = 128 GDN decode at batch 1 (fp32 state, merge interval 16).  Inputs are the
seeded synthetic ones from ``workloads`` and sit in device memory before the
timed region; W untimed steps precede K timed ones, bracketed by device
synchronization.  K is rounded up to whole merge cycles of every rotated pool
(``steps`` in the line; the requested count is ``steps_requested``), so the
timed window holds the append/merge mix of the cycle.  In graph mode the K
steps are one captured graph, replayed once untimed and then five times, each
timed replay bracketed by its own event pair and preceded by an untimed replay
already queued ahead of it (so the timed one starts back to back, as a decode
loop's steps do); the median timed replay is reported.

Output: the last stdout line is one compact JSON object (a few KB): the
headline, its ``roofline``, ``cpu_baseline``, the eager baseline and one short
row per other workload.  Every measured row in full goes to stderr as it is
taken, and to ``--detail FILE`` when given.

``roofline`` describes the decode kernel: algorithmic bytes per launch (the
traffic model in ``linear_attention_recurrent_dl_amd.traffic`` summed over the
entries of each launch with their actual live-log lengths) divided by the
average launch duration, measured with HIP events recorded on the stream the
kernel runs on.  ``workloads`` repeats the measurement for the plain
linear-attention workload (batch 1, d = 16: latency only), the batch >= 64
workloads and the eager baseline; at batch >= 64 several independent pools (layers)
are decoded in rotation so that the working set exceeds the 256 MB Infinity
Cache and the bytes come from HBM.  ``cpu_baseline`` times the fp64 oracle on
the host on a bounded sample of the headline workload.

``--sweep merge`` measures the merge interval M in {2, 4, 8, 16, 32, 64} at
batch 128, d = 128, fp32 state, for each operator family (plain, GDN, GLA-style,
KDA-style), with the eager kernel (M = 1) as reference, on cold rotated pools.
``--sweep state`` decodes one pool of 128 MiB to 1 GiB (B = 64 .. 512, d = 128,
fp32) per family (GDN, KDA-style, GLA-style) without rotation, DeltaLog and
eager, so that the Infinity Cache shows.  ``--sweep split`` compares fused
replay with split ReplayPrep by batch and value-tile width.  ``--sweep stream``
times the read-only streaming reference over grid shapes (one round of blocks
against several rounds).  Each prints one JSON line of rows instead of the
headline line.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "linear_attention_recurrent_dl_amd", "csrc")


def kernel_source_hash() -> str:
    from linear_attention_recurrent_dl_amd.rocprof_summary import kernel_source_hash as ksh
    return ksh()


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="2",
                    help="headline workload: config index 1-5, gB = GDN fp32 d=128 at batch B, kB = config 4 at batch B")
    ap.add_argument("--rotate", type=int, default=1, help="independent pools decoded in rotation (headline)")
    ap.add_argument("--value-tile", type=int, default=0,
                    help="value-tile width B_V for the headline pools (0 = library default)")
    ap.add_argument("--no-extra", action="store_true", help="skip the batch >= 64 workloads")
    ap.add_argument("--extra", default="1,3,4,5,5tp8,g64,g128,g256,g512",
                    help="comma list of extra workloads (config index or gB = GDN fp32 at batch B)")
    ap.add_argument("--extra-steps", type=int, default=0,
                    help="timed steps per extra workload (0 = whole merge cycles of every rotated pool, at least 4 L)")
    ap.add_argument("--no-eager", action="store_true", help="skip the eager baseline runs")
    ap.add_argument("--rotate-bytes", type=float, default=1.25 * 2 ** 30,
                    help="minimum bytes of pools rotated per extra workload (cold cache)")
    ap.add_argument("--no-graph", action="store_true", help="launch mode only (no HIP-graph replay)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--distinct-steps", type=int, default=0,
                    help="distinct input steps staged per workload (0 = min(steps, 4 cycles))")
    ap.add_argument("--flush", default="g256,4",
                    help="comma list of workloads whose full logs dl_flush_all materializes ('' = none)")
    ap.add_argument("--windows", default="2:16,2:64,2:256,g128:16,g128:64",
                    help="comma list of workload:W window measurements ('' = none)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming reference (a read-only kernel of each decode launch's grid and bytes)")
    ap.add_argument("--detail", default="",
                    help="also write every measured row (headline, workloads, windows, flushes, host calls) "
                         "to this JSON file")
    ap.add_argument("--sweep", choices=["merge", "state", "split", "stream"], default=None,
                    help="merge-interval, state-size, split-replay or streaming-reference sweep instead of the "
                         "headline line")
    return ap.parse_args(argv)


# --------------------------------------------------------------------------
class Staged:
    """A workload's pools and device-resident step inputs, ready to launch."""

    def __init__(self, cfg, eager: bool, rotate: int, distinct: int, torch, dl, native, value_tile: int = 0,
                 replay_split: bool = False):
        from workloads import Workload
        from linear_attention_recurrent_dl_amd import traffic

        self.cfg, self.eager, self.R = cfg, eager, rotate
        self.torch, self.N = torch, native
        self.lib = native.lib()
        wl = Workload(cfg)
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
        st, it = tdt[cfg.state_dtype], tdt[cfg.in_dtype]
        L = 1 if eager else cfg.L
        self.L = L
        self.shape = traffic.StepShape(cfg.H_v, cfg.H_k, cfg.d, cfg.d, cfg.decay, cfg.update,
                                       cfg.state_dtype, cfg.in_dtype, L)
        self.pools = [dl.DeltaLogPool(cfg.num_slots, cfg.H_v, cfg.H_k, cfg.d, L, cfg.decay, cfg.update,
                                      cfg.state_dtype, cfg.in_dtype, max_batch=cfg.batch,
                                      value_tile=value_tile, replay_split=replay_split and not eager)
                      for _ in range(rotate)]
        self.value_tile = self.pools[0].value_tile
        self.shadow = [dl.DeltaLogPool(cfg.num_slots, cfg.H_v, cfg.H_k, cfg.d, L, cfg.decay, cfg.update,
                                       cfg.state_dtype, cfg.in_dtype, max_batch=cfg.batch, device=None)
                       for _ in range(rotate)]
        # initial states: every slot's seeded base, copied to all rotated pools
        for lo in range(0, cfg.num_slots, cfg.batch):
            ids = np.arange(lo, min(cfg.num_slots, lo + cfg.batch), dtype=np.int32)
            init = torch.from_numpy(wl.init_base(ids)).to("cuda").to(st).contiguous()
            for p, sp in zip(self.pools, self.shadow):
                p.assign(ids, init)
                sp.assign(ids)
            del init
        self.bank = None
        if cfg.replace_per_step:
            self.bank = torch.from_numpy(wl.bank_states()).to("cuda").to(st).contiguous()
        # ragged initial fill (serving pool): decode the fill steps, untimed
        fill = wl.fill_steps()
        for inp in wl.generate(fill):
            self._decode_inputs_now(inp, it)
        descs = wl.main_steps(distinct)
        self.inputs = []
        for inp in wl.generate(descs):
            d = {"ids": np.ascontiguousarray(inp.slot_ids, dtype=np.int32),
                 "q": torch.from_numpy(inp.q).to("cuda").to(it).contiguous(),
                 "k": torch.from_numpy(inp.k).to("cuda").to(it).contiguous(),
                 "v": torch.from_numpy(inp.v).to("cuda").to(it).contiguous(),
                 "lam": None if inp.lam is None else torch.from_numpy(inp.lam).to("cuda"),
                 "beta": None if inp.beta is None else torch.from_numpy(inp.beta).to("cuda"),
                 "out": torch.empty((inp.batch, cfg.H_v, cfg.d), dtype=torch.float32, device="cuda"),
                 "rep": np.ascontiguousarray(inp.replace_ids, dtype=np.int32),
                 "rep_src": None}
            if len(inp.replace_ids):
                # bank entries are contiguous: the fresh states start at this offset
                d["rep_src"] = self.bank[int(inp.replace_bank[0]):].data_ptr()
            d["args"] = self._args(d)
            self.inputs.append(d)
        torch.cuda.synchronize()

    def _decode_inputs_now(self, inp, it):
        torch = self.torch
        q = torch.from_numpy(inp.q).to("cuda").to(it).contiguous()
        k = torch.from_numpy(inp.k).to("cuda").to(it).contiguous()
        v = torch.from_numpy(inp.v).to("cuda").to(it).contiguous()
        lam = None if inp.lam is None else torch.from_numpy(inp.lam).to("cuda")
        beta = None if inp.beta is None else torch.from_numpy(inp.beta).to("cuda")
        for p, sp in zip(self.pools, self.shadow):
            if self.eager:
                p.eager_step(inp.slot_ids, q, k, v, lam, beta)
            else:
                p.decode_step(inp.slot_ids, q, k, v, lam, beta)
            sp.decode_step(inp.slot_ids)

    def _args(self, d):
        ids = d["ids"]
        return (len(ids), ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), d["q"].data_ptr(),
                d["k"].data_ptr(), d["v"].data_ptr(),
                None if d["lam"] is None else d["lam"].data_ptr(),
                None if d["beta"] is None else d["beta"].data_ptr(), d["out"].data_ptr())

    def plan_bytes(self, t0: int, count: int):
        """Algorithmic decode bytes of steps t0 .. t0+count-1, from the host-only
        shadow pools (same call sequence, nothing launched)."""
        from linear_attention_recurrent_dl_amd import traffic
        total = 0.0
        assign_total = 0.0
        for t in range(t0, t0 + count):
            d = self.inputs[t % len(self.inputs)]
            sp = self.shadow[t % self.R]
            if len(d["rep"]):
                sp.assign(d["rep"])
                assign_total += len(d["rep"]) * self.cfg.H_v * traffic.assign_head_bytes(self.shape)
            if self.eager:
                total += len(d["ids"]) * self.cfg.H_v * traffic.eager_head_step_bytes(self.shape)
            else:
                _, idx = sp.schedule(d["ids"])
                total += self.cfg.H_v * sum(traffic.deltalog_head_step_bytes(self.shape, int(n)) for n in idx)
            sp.decode_step(d["ids"])
        return total, assign_total

    def run(self, t0: int, count: int, events=None, decode: bool = True):
        """Launch steps t0 .. t0+count-1 on the current stream (decode=False:
        only their fresh-slot assignments)."""
        torch = self.torch
        stream = torch.cuda.current_stream().cuda_stream
        dec = self.lib.dl_eager_step if self.eager else self.lib.dl_decode_step
        asg = self.lib.dl_slot_assign
        for t in range(t0, t0 + count):
            d = self.inputs[t % len(self.inputs)]
            pool = self.pools[t % self.R]
            if len(d["rep"]):
                rc = asg(pool.handle, len(d["rep"]), d["rep"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                         d["rep_src"], stream)
                if rc:
                    self.N.check(rc, "dl_slot_assign")
            if not decode:
                continue
            if events is not None:
                events[t - t0][0].record()
            rc = dec(pool.handle, *d["args"], stream)
            if rc:
                self.N.check(rc, "decode")
            if events is not None:
                events[t - t0][1].record()

    def close(self):
        for p in self.pools:
            p.close()
        self.pools = []
        self.inputs = []
        self.bank = None


def cycle_steps(rotate: int, L: int, at_least: int) -> int:
    """Timed steps for `rotate` pools decoded in turn: a whole number of merge
    cycles of every pool (rotate * L steps each), and at least `at_least`, so
    that every measurement window holds the same mix of append and merge steps."""
    per = rotate * L
    return per * max(1, -(-at_least // per))


def time_workload(cfg, eager, steps, warmup, rotate, distinct, torch, dl, native, value_tile=0, graph=True,
                  replay_split=False, reps=5):
    """Launch mode: W warm-up steps, then K steps each bracketed by a HIP event
    pair on the launch stream.  Graph mode: the next K steps captured once in a
    HIP graph (the kernels read the live-log lengths on the device, so the
    capture stays valid for every replay), replayed once untimed, then `reps`
    times, each timed by an event pair around the replay; the median counts."""
    st = Staged(cfg, eager, rotate, distinct, torch, dl, native, value_tile, replay_split)
    try:
        st.plan_bytes(0, warmup)                 # advance the shadow schedule past warm-up
        st.run(0, warmup)
        torch.cuda.synchronize()
        dec_bytes, asg_bytes = st.plan_bytes(warmup, steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        t_start.record()
        st.run(warmup, steps, ev)
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        out = dict(total_ms=t_start.elapsed_time(t_end), wall_s=wall,
                   launch_ms=[a.elapsed_time(b) for a, b in ev], dec_bytes=dec_bytes,
                   asg_bytes=asg_bytes, L=st.L, value_tile=st.value_tile, steps=steps)
        if graph:
            S = steps
            t0 = warmup + steps
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st.run(t0, S)
            st.plan_bytes(t0, S)                 # the warm-up replay
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            times = []
            for _ in range(max(1, reps)):
                # an untimed replay runs ahead of the timed one, so that the
                # timed replay's launch is already queued when its first
                # kernel may start: the events bracket exactly S steps of
                # back-to-back decode, as in a decode loop
                torch.cuda.synchronize()
                st.plan_bytes(t0, S)
                g.replay()
                gb_dec, gb_asg = st.plan_bytes(t0, S)    # every replay covers the same whole cycles
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            out["graph"] = dict(ms=float(np.median(times)), replay_ms=times, steps=S, dec_bytes=gb_dec,
                                asg_bytes=gb_asg)
            del g
            if gb_asg > 0:
                # the same steps' assignments alone: their replay time is taken
                # off, leaving the decode launches' share of the step
                ga = torch.cuda.CUDAGraph()
                with torch.cuda.graph(ga):
                    st.run(t0, S, decode=False)
                ga.replay()
                torch.cuda.synchronize()
                atimes = []
                for _ in range(max(1, reps)):
                    ga.replay()                  # untimed, ahead of the timed replay (as above)
                    e0.record()
                    ga.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    atimes.append(e0.elapsed_time(e1))
                out["graph"]["assign_ms"] = float(np.median(atimes))
                del ga
        return out
    finally:
        st.close()
        torch.cuda.empty_cache()


def time_window(cfg, W, rotate, torch, dl, native, reps: int = 4, graph: bool = True):
    """W steps of the workload's first batch of slots in one window launch per
    pool, rotating over `rotate` pools (cold cache when their bytes exceed the
    Infinity Cache).  The timed region is one graph replay of `reps` launches
    per pool, after an untimed replay (graph=False: the same launches issued
    directly, after one untimed round), median of three timed rounds; inputs
    are device resident."""
    from linear_attention_recurrent_dl_amd import traffic
    from workloads import Workload
    wl = Workload(cfg)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    st, it = tdt[cfg.state_dtype], tdt[cfg.in_dtype]
    pools = [dl.DeltaLogPool(cfg.num_slots, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update,
                             cfg.state_dtype, cfg.in_dtype, max_batch=cfg.batch) for _ in range(rotate)]
    try:
        for lo in range(0, cfg.num_slots, cfg.batch):
            ids = np.arange(lo, min(cfg.num_slots, lo + cfg.batch), dtype=np.int32)
            init = torch.from_numpy(wl.init_base(ids)).to("cuda").to(st).contiguous()
            for p in pools:
                p.assign(ids, init)
            del init
        steps = wl.generate(wl.main_steps(W))
        ids = np.ascontiguousarray(steps[0].slot_ids, dtype=np.int32)

        def stack(name, dt):
            xs = [getattr(s_, name) for s_ in steps]
            return None if xs[0] is None else torch.from_numpy(np.stack(xs)).to("cuda").to(dt).contiguous()

        q, k, v = stack("q", it), stack("k", it), stack("v", it)
        lam, beta = stack("lam", torch.float32), stack("beta", torch.float32)
        out = torch.empty((W, len(ids), cfg.H_v, cfg.d), dtype=torch.float32, device="cuda")
        for p in pools:                          # first window: empties the logs
            p.decode_window(ids, W, q, k, v, lam, beta, out)
        torch.cuda.synchronize()

        def launches():
            for _ in range(reps):
                for p in pools:
                    p.decode_window(ids, W, q, k, v, lam, beta, out)

        g = None
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                launches()
        run = g.replay if graph else launches
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(3):
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        launches = reps * rotate
        us = float(np.median(times)) * 1e3 / launches
        sh = traffic.StepShape(cfg.H_v, cfg.H_k, cfg.d, cfg.d, cfg.decay, cfg.update, cfg.state_dtype,
                               cfg.in_dtype, cfg.L)
        bpl = len(ids) * cfg.H_v * traffic.window_head_bytes(sh, W)
        del g
        return {"workload": cfg.name, "kernel": "dl_window_kernel", "W": W, "batch": len(ids),
                "rotated_pools": rotate, "value_tile": pools[0].value_tile,
                "timing": "graph replay" if graph else "direct launches",
                "launch_us": us, "us_per_step": us / W,
                "head_steps_per_s": len(ids) * cfg.H_v * W / (us * 1e-6),
                "tokens_per_s": len(ids) * W / (us * 1e-6),
                "bytes_per_launch": bpl, "GBps": bpl / (us * 1e-6) / 1e9,
                "frac_of_8TBps": bpl / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    finally:
        for p in pools:
            p.close()
        torch.cuda.empty_cache()


def time_flush(cfg, rotate, torch, dl, native, reps: int = 5):
    """dl_flush_all on pools whose every log is full (L - 1 entries): the
    standalone merge materializes base + log and empties the log.  Each timed
    round refills the logs with L - 1 untimed decode steps, then one graph
    replay flushes every pool; median of `reps` rounds."""
    from linear_attention_recurrent_dl_amd import traffic
    st = Staged(cfg, False, rotate, cfg.L - 1, torch, dl, native)
    try:
        C = cfg.L - 1
        st.run(0, C * rotate)                     # every slot of every pool holds L - 1 live entries
        torch.cuda.synchronize()
        # flush_all picks its slots from the host mirror, which is full here; the
        # capture empties the mirror while the device logs stay full for the replay
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for p in st.pools:
                p.flush_all()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for rep in range(reps):
            if rep:
                st.run(0, C * rotate)             # refill: mirror and device back to L - 1 entries
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        us = float(np.median(times)) * 1e3 / rotate
        sh = traffic.StepShape(cfg.H_v, cfg.H_k, cfg.d, cfg.d, cfg.decay, cfg.update, cfg.state_dtype,
                               cfg.in_dtype, cfg.L)
        bpl = cfg.num_slots * cfg.H_v * traffic.merge_head_bytes(sh, C)
        return {"workload": cfg.name, "kernel": "dl_step_kernel (standalone merge)", "live_entries": C,
                "slots": cfg.num_slots, "rotated_pools": rotate, "launch_us": us, "bytes_per_launch": bpl,
                "GBps": bpl / (us * 1e-6) / 1e9, "frac_of_8TBps": bpl / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                "replays_ms": times}
    finally:
        st.close()
        torch.cuda.empty_cache()


def host_call_cost(dl, native, seconds: float = 0.5):
    """Host-side cost of one dl_decode_step call (validation, duplicate check,
    live-length mirror; the phase split of every entry), measured on host-only
    pools, which do everything but enqueue: microseconds per call through the
    C symbol (ctypes, whose conversion of the ten arguments is included), for
    batches of 1, 64 and 256 slots."""
    from workloads import headline_gdn
    lib = native.lib()
    out = []
    for B in (1, 64, 256):
        c = headline_gdn(B)
        pool = dl.DeltaLogPool(c.num_slots, c.H_v, c.H_k, c.d, c.L, c.decay, c.update, c.state_dtype,
                               c.in_dtype, max_batch=B, device=None)
        ids = np.arange(B, dtype=np.int32)
        ip = ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        f, h = lib.dl_decode_step, pool.handle
        n, t0 = 0, time.perf_counter()
        while True:
            for _ in range(1000):
                f(h, B, ip, None, None, None, None, None, None, None)
            n += 1000
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        pool.close()
        out.append({"batch": B, "us_per_call": el / n * 1e6, "calls": n})
    # the Python-to-C call itself: a trivial exported function in the same loop
    g, n, t0 = lib.dl_launch_slot_limit, 0, time.perf_counter()
    while True:
        for _ in range(1000):
            g()
        n += 1000
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    floor = el / n * 1e6
    for o in out:
        o["trivial_call_us"] = floor          # a no-argument exported function, same path
    return out


def summarize(cfg, r, steps, tag):
    from linear_attention_recurrent_dl_amd import traffic
    sh = traffic.StepShape(cfg.H_v, cfg.H_k, cfg.d, cfg.d, cfg.decay, cfg.update, cfg.state_dtype,
                           cfg.in_dtype, r["L"])
    launch_ms = float(np.mean(r["launch_ms"]))
    bytes_per_launch = r["dec_bytes"] / steps
    res = {
        "workload": cfg.name, "kernel": tag, "batch": cfg.batch, "H_v": cfg.H_v, "H_k": cfg.H_k,
        "d": cfg.d, "L": r["L"], "state": cfg.state_dtype, "value_tile": r["value_tile"],
        "decode_bytes_per_launch": bytes_per_launch,
        "model_bytes_per_head_step": (traffic.eager_head_step_bytes(sh) if tag == "eager"
                                      else traffic.deltalog_model_bytes(sh)),
        "assign_bytes_per_step": r["asg_bytes"] / steps,
        # launch mode: one host call per step, an event pair around every launch
        "launch_mode": {
            "ms_per_step": r["total_ms"] / steps,
            "head_steps_per_s": cfg.batch * cfg.H_v * steps / (r["total_ms"] * 1e-3),
            "decode_event_pair_us_avg": launch_ms * 1e3,
            "decode_event_pair_us_median": float(np.median(r["launch_ms"])) * 1e3,
            "decode_GBps_event_pair": bytes_per_launch / (launch_ms * 1e-3) / 1e9,
        },
    }
    gr = r.get("graph")
    if gr:
        ms_step = gr["ms"] / gr["steps"]
        res.update({
            "ms_per_step": ms_step,
            "graph_replays_ms": [round(x, 5) for x in gr["replay_ms"]],
            "head_steps_per_s": cfg.batch * cfg.H_v * gr["steps"] / (gr["ms"] * 1e-3),
            "tokens_per_s": cfg.batch * gr["steps"] / (gr["ms"] * 1e-3),
        })
        if gr["asg_bytes"] == 0:
            # a step is exactly one decode launch: graph time per step is its duration
            dec_us = ms_step * 1e3
            res["decode_launch_us"] = dec_us
            res["decode_launch_source"] = "graph replay, back-to-back launches"
            bpl = gr["dec_bytes"] / gr["steps"]
            res["decode_bytes_per_launch"] = bpl
        else:
            # a step is assignments + one decode launch: the decode's share is
            # the step's replay time minus that of the assignments alone
            dec_us = (gr["ms"] - gr["assign_ms"]) / gr["steps"] * 1e3
            res["decode_launch_us"] = dec_us
            res["decode_launch_source"] = "graph replay minus an assignment-only replay of the same steps"
            res["assign_us_per_step"] = gr["assign_ms"] / gr["steps"] * 1e3
            bpl = gr["dec_bytes"] / gr["steps"]
            res["decode_bytes_per_launch"] = bpl
    else:
        res.update({"ms_per_step": r["total_ms"] / steps,
                    "head_steps_per_s": res["launch_mode"]["head_steps_per_s"],
                    "tokens_per_s": cfg.batch * steps / (r["total_ms"] * 1e-3)})
        dec_us = launch_ms * 1e3
        res["decode_launch_us"] = dec_us
        res["decode_launch_source"] = "event pair per launch"
        bpl = bytes_per_launch
    res["decode_GBps"] = bpl / (dec_us * 1e-6) / 1e9
    res["decode_frac_of_8TBps"] = res["decode_GBps"] / PEAK_HBM_GBS
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, seconds: float):
    """fp64 oracle (eager recurrence) on a bounded sample of the workload."""
    import oracle
    from workloads import Workload
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    wl = Workload(cfg)
    ids = np.arange(cfg.num_slots, dtype=np.int32)
    E = oracle.EagerPool(ids, cfg.H_v, cfg.d, cfg.d, cfg.decay, cfg.update, init=wl.init_base(ids))
    inputs = wl.generate(wl.main_steps(min(cfg.steps, 64)))
    E.step(inputs[0].slot_ids, inputs[0].q, inputs[0].k, inputs[0].v, inputs[0].lam, inputs[0].beta)
    n, w0, c0 = 0, time.perf_counter(), time.process_time()
    while True:
        inp = inputs[(n + 1) % len(inputs)]
        E.step(inp.slot_ids, inp.q, inp.k, inp.v, inp.lam, inp.beta)
        n += 1
        el = time.perf_counter() - w0
        if (el >= seconds and n >= 32) or el >= 3 * seconds:
            break
    wall = time.perf_counter() - w0
    cpu = time.process_time() - c0
    return {"value": cfg.batch * cfg.H_v * n / wall, "unit": "head-steps/s",
            "cores": max(1, int(round(cpu / wall))), "kind": "oracle",
            "sample": f"{n} steps of {cfg.name} (all {cfg.batch * cfg.H_v} slot-heads each), fp64 NumPy "
                      f"eager recurrence, {wall:.1f} s wall",
            "tokens_per_s": cfg.batch * n / wall, "cpu_seconds": cpu, "blas_threads": blas_threads,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}


def stream_reference(torch, mib: int = 1024, reps: int = 10):
    """Device bandwidth of plain streaming kernels on this GPU (context for the
    roofline): a 1 GiB copy (read + write) and a read-only reduction."""
    n = mib << 20
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    a.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    e0.record()
    for _ in range(reps):
        a.sum()
    e1.record()
    torch.cuda.synchronize()
    read_gbs = n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": copy_gbs, "read_GBps": read_gbs, "bytes": n, "kernels": "torch copy_ / sum"}


_PROBE = None


def _probe_lib():
    global _PROBE
    if _PROBE is None:
        path = os.path.join(ROOT, "linear_attention_recurrent_dl_amd", "libdl_stream_probe.so")
        lib = ctypes.CDLL(path)
        lib.dl_probe_stream_read.restype = ctypes.c_int
        lib.dl_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_uint32, ctypes.c_void_p]
        _PROBE = lib
    return _PROBE


def stream_ceiling(torch, blocks: int, threads: int, bytes_per_launch: float, rotate: int, reps: int = 5):
    """A read-only kernel with the decode launch's grid (blocks x threads),
    each block reading its own contiguous share of bytes_per_launch with the
    same 16-byte non-temporal loads, over `rotate` rotated buffers like the
    workload's pools: how fast this GPU moves those bytes in that grid with no
    other work.  Graph of back-to-back launches, median of `reps` replays."""
    lib = _probe_lib()
    unit = threads * 16
    block_bytes = int(max(unit, -(-int(bytes_per_launch / blocks) // unit) * unit))
    total = block_bytes * blocks
    bufs = [torch.ones(total // 4, dtype=torch.float32, device="cuda") for _ in range(rotate)]
    dst = torch.empty(blocks * threads, dtype=torch.float32, device="cuda")
    per = max(1, -(-64 // rotate))

    def launches():
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(per):
            for b in bufs:
                rc = lib.dl_probe_stream_read(b.data_ptr(), dst.data_ptr(), blocks, threads, block_bytes, stream)
                if rc:
                    raise RuntimeError(f"stream probe launch failed ({rc})")

    launches()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launches()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    us = float(np.median(times)) * 1e3 / (per * rotate)
    del g, bufs, dst
    torch.cuda.empty_cache()
    return {"blocks": blocks, "threads": threads, "block_bytes": block_bytes, "bytes": total, "rotated": rotate,
            "us": us, "GBps": total / (us * 1e-6) / 1e9}


def decode_kernel(cfg, value_tile: int) -> str:
    """Name of the kernel a decode step of the workload runs: the launcher's
    rule for the one-barrier narrow-tile kernel (tiles of at most 32 columns,
    scalar or no decay, at least four 16-byte key chunks per log entry, every
    row group owning a tile row, at most 32 bytes of value-side factor per
    lane), the general kernel otherwise."""
    isz = 2 if cfg.in_dtype == "bf16" else 4
    ssz = 2 if cfg.state_dtype == "bf16" else 4
    bsz = 4 if cfg.update == "delta" else isz            # b is kept in fp32 for the delta rule
    cpe = cfg.d // (16 // isz)                           # 16-byte chunks per key
    threads = 256 if cfg.d >= 128 else (128 if cfg.d >= 64 else 64)
    col_groups = max(1, value_tile // (16 // ssz))
    ragged = threads // col_groups > cfg.d
    if (value_tile <= 32 and cfg.decay != "per_key" and cpe >= 4 and not ragged
            and (value_tile // (cpe // 2)) * bsz <= 32):
        return "dl_small_kernel"
    return "dl_step_kernel"


def decode_grid(cfg, value_tile: int):
    """(blocks, threads) of one decode launch of the workload."""
    threads = 256 if cfg.d >= 128 else (128 if cfg.d >= 64 else 64)
    return min(cfg.batch, 512) * cfg.H_v * (cfg.d // value_tile), threads


def attach_ceiling(row, cfg, torch, rotate):
    """Add the streaming reference for a measured DeltaLog row: same grid,
    same algorithmic bytes per launch."""
    blocks, threads = decode_grid(cfg, row["value_tile"])
    c = stream_ceiling(torch, blocks, threads, row["decode_bytes_per_launch"], rotate)
    row["stream_ceiling"] = c
    row["frac_of_stream_ceiling"] = row["decode_GBps"] / c["GBps"]
    return row


def pool_bytes(dl, c, L=None) -> int:
    return sum(dl.dl_pool_sizes(dl.make_desc(c.num_slots, c.batch, c.H_v, c.H_k, c.d, L or c.L, c.decay,
                                             c.update, c.state_dtype, c.in_dtype)))


def sweep_row(c, eager, R, torch, dl, native, graph=True, value_tile=0, replay_split=False):
    L = 1 if eager else c.L
    steps = cycle_steps(R, L, max(4 * L, 64))
    r = time_workload(c, eager, steps, L, R, min(4 * L, steps + L, 64), torch, dl, native, graph=graph,
                      value_tile=value_tile, replay_split=replay_split)
    s = summarize(c, r, steps, "eager" if eager else ("deltalog-split" if replay_split else "deltalog"))
    s["rotated_pools"] = R
    s["pool_bytes"] = pool_bytes(dl, c, L)
    return s


def run_sweep(kind, a, torch, dl, native) -> dict:
    """Merge-interval or state-size sweep (see the module docstring)."""
    from workloads import SWEEP_OPERATORS, headline_gdn, merge_sweep_config
    rows = []

    def brief(s, **kw):
        row = {k: s[k] for k in ("workload", "kernel", "batch", "L", "value_tile", "decode_launch_us",
                                 "decode_GBps", "decode_frac_of_8TBps", "head_steps_per_s",
                                 "model_bytes_per_head_step", "rotated_pools", "pool_bytes")}
        row.update(kw)
        print(f"[sweep] {json.dumps(row)}", file=sys.stderr, flush=True)
        return row

    if kind == "merge":
        for op in SWEEP_OPERATORS:
            ref = merge_sweep_config(op, 16)
            R = max(1, int(np.ceil(a.rotate_bytes / pool_bytes(dl, ref, 1))))
            eager = brief(sweep_row(ref, True, R, torch, dl, native), op=op, M=1)
            rows.append(eager)
            for M in (2, 4, 8, 16, 32, 64):
                c = merge_sweep_config(op, M)
                try:
                    ws = pool_bytes(dl, c)
                except dl.DeltaLogError as err:
                    rows.append({"op": op, "M": M, "workload": c.name, "unsupported": str(err)})
                    print(f"[sweep] {op} M={M}: {err}", file=sys.stderr, flush=True)
                    continue
                R = max(1, int(np.ceil(a.rotate_bytes / ws)))
                s = sweep_row(c, False, R, torch, dl, native)
                rows.append(brief(s, op=op, M=M, vs_eager=eager["decode_launch_us"] / s["decode_launch_us"]))
    elif kind == "split":
        # fused replay (every tile unit recomputes its slot-head's coefficients)
        # against split ReplayPrep, by batch and tile width
        for op, mk in (("gdn", lambda B: headline_gdn(B)), ("kda", lambda B: merge_sweep_config("kda", 16, B))):
            for B, tiles in ((1, (32, 16)), (64, (128, 64, 32)), (128, (128, 64, 32))):
                c = mk(B)
                R = max(1, int(np.ceil(a.rotate_bytes / pool_bytes(dl, c)))) if B > 1 else 1
                for bv in tiles:
                    fu = brief(sweep_row(c, False, R, torch, dl, native, value_tile=bv), op=op, B_V=bv)
                    sp = brief(sweep_row(c, False, R, torch, dl, native, value_tile=bv, replay_split=True),
                               op=op, B_V=bv)
                    sp["split_vs_fused"] = fu["decode_launch_us"] / sp["decode_launch_us"]
                    rows += [fu, sp]
    elif kind == "stream":
        # the read-only reference kernel over grid shapes: one round of blocks
        # against several rounds, at the decode launches' block sizes
        shapes = [(2048, 128, 16 << 10), (2048, 128, 24 << 10), (4096, 128, 24 << 10), (8192, 128, 24 << 10),
                  (256, 256, 8 << 10), (2048, 256, 72 << 10), (4096, 256, 72 << 10), (8192, 256, 72 << 10),
                  (8192, 256, 40 << 10), (16384, 256, 256 << 10)]
        for blocks, threads, bb in shapes:
            total = blocks * bb
            R = 1 if total >= a.rotate_bytes else int(np.ceil(a.rotate_bytes / total))
            c = stream_ceiling(torch, blocks, threads, blocks * bb, R)
            c["frac_of_8TBps"] = c["GBps"] / PEAK_HBM_GBS
            print(f"[sweep] {json.dumps(c)}", file=sys.stderr, flush=True)
            rows.append(c)
    else:
        for op in ("gdn", "kda", "gla"):
            for B in (64, 128, 256, 512):
                c = headline_gdn(B) if op == "gdn" else merge_sweep_config(op, 16, B)
                mib = B * c.H_v * c.d * c.d * 4 / 2 ** 20
                dls = brief(sweep_row(c, False, 1, torch, dl, native), op=op, base_MiB=mib)
                eg = brief(sweep_row(c, True, 1, torch, dl, native), op=op, base_MiB=mib)
                dls["vs_eager"] = eg["decode_launch_us"] / dls["decode_launch_us"]
                rows += [dls, eg]
    return {"sweep": kind, "unit": "us per decode step; GB/s of algorithmic bytes",
            "peak_GBps": PEAK_HBM_GBS, "rows": rows, "kernel_source_hash": kernel_source_hash()}


def extra_cfg(tag: str):
    """Config index 1-5; gB = GDN fp32 d = 128 at batch B; kB = config 4
    (KDA-style) at batch B; NtpG = config N's per-GPU share under G-way head
    sharding (H_v / G v-heads, H_k / G q/k heads)."""
    import dataclasses
    from workloads import CONFIGS, headline_gdn
    if tag.startswith("g"):
        return headline_gdn(int(tag[1:]))
    if tag.startswith("k"):
        B = int(tag[1:])
        return dataclasses.replace(CONFIGS[4], index=200 + B, name=f"kda_b{B}_h32_d128", num_slots=B, batch=B,
                                   seed=CONFIGS[4].seed + B)
    if "tp" in tag:
        idx, G = (int(x) for x in tag.split("tp"))
        base = CONFIGS[idx]
        return dataclasses.replace(base, H_v=base.H_v // G, H_k=max(1, base.H_k // G),
                                   name=f"{base.name}_tp{G}_share")
    return CONFIGS[int(tag)]


def main(argv=None) -> int:
    a = parse(argv)
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU per process; --gpus must be 1",
                          "requested_gpus": a.gpus}))
        print("bench.py: only --gpus 1 is supported (one GPU per process, no multi-GPU path)",
              file=sys.stderr)
        return 2
    import torch

    import linear_attention_recurrent_dl_amd as dl
    from linear_attention_recurrent_dl_amd import _native as native
    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    native.lib()
    torch.cuda.set_device(0)
    if a.sweep:
        print(json.dumps(run_sweep(a.sweep, a, torch, dl, native)), flush=True)
        return 0
    cfg = extra_cfg(a.workload)
    # whole merge cycles of every rotated pool, so the timed window holds the
    # cycle's own mix of append and merge steps
    steps, warmup = cycle_steps(a.rotate, cfg.L, max(1, a.steps)), a.warmup
    distinct = a.distinct_steps or min(steps + warmup, 4 * cfg.L)
    print(f"[bench] headline {cfg.describe()} steps={steps} warmup={warmup}", file=sys.stderr, flush=True)

    if a.calib_copy_mib:
        src = torch.empty(a.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream_ref = stream_reference(torch)
    print(f"[bench] stream reference {json.dumps(stream_ref)}", file=sys.stderr, flush=True)
    r = time_workload(cfg, False, steps, warmup, a.rotate, distinct, torch, dl, native, a.value_tile,
                      graph=not a.no_graph)
    head = summarize(cfg, r, steps, "deltalog")
    if not a.no_ceiling:
        attach_ceiling(head, cfg, torch, a.rotate)
    print(f"[bench] {json.dumps(head)}", file=sys.stderr, flush=True)
    eager_head = None
    if not a.no_eager:
        re_ = time_workload(cfg, True, steps, warmup, a.rotate, distinct, torch, dl, native, a.value_tile,
                            graph=not a.no_graph)
        eager_head = summarize(cfg, re_, steps, "eager")
        print(f"[bench] {json.dumps(eager_head)}", file=sys.stderr, flush=True)

    extras = []
    if not a.no_extra:
        for tag in [t for t in a.extra.split(",") if t]:
            c = extra_cfg(tag)
            from linear_attention_recurrent_dl_amd import traffic
            ws = sum(dl.dl_pool_sizes(dl.make_desc(c.num_slots, c.batch, c.H_v, c.H_k, c.d, c.L, c.decay,
                                                   c.update, c.state_dtype, c.in_dtype)))
            # batch-1 workloads are latency-bound with a state of a few KiB: no rotation
            R = 1 if c.batch == 1 else max(1, int(np.ceil(a.rotate_bytes / ws)))
            xs = a.extra_steps or cycle_steps(R, c.L, 4 * c.L)
            for eager in ([False] if a.no_eager else [False, True]):
                rr = time_workload(c, eager, xs, c.L, R, min(4 * c.L, xs + c.L), torch, dl, native,
                                   graph=not a.no_graph)
                s = summarize(c, rr, xs, "eager" if eager else "deltalog")
                s["rotated_pools"] = R
                if not eager and not a.no_ceiling:
                    attach_ceiling(s, c, torch, R)
                s["pool_bytes"] = ws if not eager else sum(dl.dl_pool_sizes(dl.make_desc(
                    c.num_slots, c.batch, c.H_v, c.H_k, c.d, 1, c.decay, c.update, c.state_dtype, c.in_dtype)))
                extras.append(s)
                print(f"[bench] {json.dumps(s)}", file=sys.stderr, flush=True)

    flushes = []
    for tag in [t for t in a.flush.split(",") if t]:
        c = extra_cfg(tag)
        R = max(1, int(np.ceil(a.rotate_bytes / pool_bytes(dl, c))))
        fr = time_flush(c, R, torch, dl, native)
        flushes.append(fr)
        print(f"[bench] flush {json.dumps(fr)}", file=sys.stderr, flush=True)

    windows = []
    for spec in [t for t in a.windows.split(",") if t]:
        tag, W = spec.split(":")
        c = extra_cfg(tag)
        R = 1 if c.batch == 1 else max(1, int(np.ceil(a.rotate_bytes / pool_bytes(dl, c))))
        wr = time_window(c, int(W), R, torch, dl, native, graph=not a.no_graph)
        step_us = {x["workload"]: x["decode_launch_us"] for x in extras if x["kernel"] == "deltalog"}
        step_us[cfg.name] = head["decode_launch_us"]
        if c.name in step_us:
            wr["decode_step_us"] = step_us[c.name]
            wr["speedup_per_step_vs_decode"] = step_us[c.name] / wr["us_per_step"]
        windows.append(wr)
        print(f"[bench] window {json.dumps(wr)}", file=sys.stderr, flush=True)

    host_cost = host_call_cost(dl, native)
    print(f"[bench] host call {json.dumps(host_cost)}", file=sys.stderr, flush=True)

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(cfg, a.cpu_seconds)
        print(f"[bench] cpu {json.dumps(cpu)}", file=sys.stderr, flush=True)

    traffic_val, traffic_src = None, None
    prof = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}_rot{a.rotate}.json")
    if os.path.exists(prof):
        try:
            with open(prof) as f:
                pj = json.load(f)
            if pj.get("kernel_source_hash") == kernel_source_hash():
                traffic_val = pj.get("hbm_bytes_per_launch")
                traffic_src = os.path.relpath(prof, ROOT)
        except Exception:
            traffic_val = None

    detail = {"headline": head, "eager_baseline": eager_head, "workloads": extras, "windows": windows,
              "flush": flushes, "host_call": host_cost, "stream_reference": stream_ref, "cpu_baseline": cpu,
              "kernel_source_hash": kernel_source_hash()}
    print(f"[bench] detail {json.dumps(detail)}", file=sys.stderr, flush=True)
    if a.detail:
        os.makedirs(os.path.dirname(os.path.abspath(a.detail)), exist_ok=True)
        with open(a.detail, "w") as f:
            json.dump(detail, f, indent=1)
    line = make_line(cfg, a.rotate, steps, warmup, a.steps, head, eager_head, extras, windows, flushes, cpu,
                     traffic_val, traffic_src, kernel_source_hash())
    print(json.dumps(line, separators=(",", ":")), flush=True)
    return 0


def line_dtype(cfg) -> str:
    """Arithmetic type of the path: the kernels compute in fp32; 16-bit state
    or inputs are widened on load (named after it)."""
    if cfg.state_dtype == "f32" and cfg.in_dtype == "f32":
        return "f32"
    return f"f32 ({cfg.state_dtype} state, {cfg.in_dtype} inputs)"


def _r(x, nd):
    return None if x is None else round(float(x), nd)


def compact_rows(extras) -> list:
    """One short row per extra workload: DeltaLog and its eager baseline side by
    side (us per decode launch, algorithmic GB/s, fraction of 8 TB/s)."""
    rows, index = [], {}
    for s in extras:
        key = s["workload"]
        if key not in index:
            index[key] = {"w": key, "B": s["batch"], "st": s["state"], "R": s.get("rotated_pools")}
            rows.append(index[key])
        row = index[key]
        if s["kernel"] == "eager":
            row["eager_us"] = _r(s["decode_launch_us"], 2)
            row["eager_GBps"] = _r(s["decode_GBps"], 0)
        else:
            row.update({"tile": s["value_tile"], "us": _r(s["decode_launch_us"], 2), "GBps": _r(s["decode_GBps"], 0),
                        "frac": _r(s["decode_frac_of_8TBps"], 3), "Mhs": _r(s["head_steps_per_s"] / 1e6, 2)})
            if "stream_ceiling" in s:
                row["ceil_GBps"] = _r(s["stream_ceiling"]["GBps"], 0)
                row["of_ceil"] = _r(s["frac_of_stream_ceiling"], 3)
    for row in rows:
        if row.get("us") and row.get("eager_us"):
            row["x_eager"] = _r(row["eager_us"] / row["us"], 3)
    return rows


def make_line(cfg, rotate, steps, warmup, steps_requested, head, eager_head, extras, windows, flushes, cpu,
              traffic_val, traffic_src, khash) -> dict:
    """The one JSON line on stdout: headline, roofline of the decode kernel,
    CPU baseline, eager baseline and one short row per other workload.  Kept
    to a few KB; the full detail goes to stderr (and --detail)."""
    line = {
        "metric": "decode head-steps/s + achieved HBM GB/s vs 8 TB/s peak, GDN h=32 d=128",
        "value": head["head_steps_per_s"],
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": steps,
        "steps_requested": steps_requested,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": line_dtype(cfg),
        "data": "synthetic (seeded)",
        "config": {"workload": cfg.name, "global_batch": cfg.batch, "v_heads": cfg.H_v, "qk_heads": cfg.H_k,
                   "d_k": cfg.d, "d_v": cfg.d, "state": cfg.state_dtype, "inputs": cfg.in_dtype,
                   "merge_interval": cfg.L, "value_tile": head["value_tile"], "rotated_pools": rotate,
                   "parallelism": "single-gpu"},
        "tokens_per_s": _r(head["tokens_per_s"], 1),
        "roofline": {"bound": "hbm", "achieved": _r(head["decode_GBps"], 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": _r(head["decode_GBps"] / PEAK_HBM_GBS, 4),
                     "traffic": traffic_val, "traffic_source": traffic_src,
                     "kernel": decode_kernel(cfg, head["value_tile"]) + " (decode, append/merge)",
                     "bytes_per_launch": _r(head["decode_bytes_per_launch"], 1),
                     "launch_us": _r(head["decode_launch_us"], 3),
                     "launch_source": head["decode_launch_source"],
                     "stream_ceiling_GBps": _r(head.get("stream_ceiling", {}).get("GBps"), 1)},
        "cpu_baseline": None if cpu is None else {
            "value": _r(cpu["value"], 1), "unit": cpu["unit"], "cores": cpu["cores"], "kind": cpu["kind"],
            "sample": cpu["sample"]},
        "eager_baseline": None if eager_head is None else {
            "us_per_step": _r(eager_head["ms_per_step"] * 1e3, 3),
            "head_steps_per_s": _r(eager_head["head_steps_per_s"], 1),
            "GBps": _r(eager_head["decode_GBps"], 1),
            "deltalog_speedup": _r(eager_head["ms_per_step"] / head["ms_per_step"], 3)},
        "workloads": compact_rows(extras),
        "windows": [{"w": w["workload"], "W": w["W"], "us_step": _r(w["us_per_step"], 3),
                     "x_decode": _r(w.get("speedup_per_step_vs_decode"), 2)} for w in windows],
        "flush": [{"w": f["workload"], "us": _r(f["launch_us"], 1), "frac": _r(f["frac_of_8TBps"], 3)}
                  for f in flushes],
        "kernel_source_hash": khash,
    }
    return line


if __name__ == "__main__":
    sys.exit(main())
