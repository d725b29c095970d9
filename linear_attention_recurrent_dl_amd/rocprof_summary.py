"""Summarize rocprofv3 output (kernel trace and PMC counters) as short text.

    python -m linear_attention_recurrent_dl_amd.rocprof_summary trace  <results.db | kernel_trace.csv>
    python -m linear_attention_recurrent_dl_amd.rocprof_summary pmc    <results.db | counter_collection.csv> COUNTER
    python -m linear_attention_recurrent_dl_amd.rocprof_summary traffic FETCH_DB WRITE_DB KERNEL_SUBSTR COPY_BYTES [OUT.json|-] [LAST_N]
    python -m linear_attention_recurrent_dl_amd.rocprof_summary tail   <kernel_trace.csv> KERNEL_SUBSTR N
    python -m linear_attention_recurrent_dl_amd.rocprof_summary phases <kernel_trace.csv> KERNEL_SUBSTR R L REPS

``trace`` prints count / average / min / max duration per kernel name;
``pmc`` prints, per kernel name, the average value of COUNTER per dispatch and
the number of dispatches.  ``traffic`` turns a FETCH_SIZE run and a
WRITE_SIZE run into HBM bytes per launch of the kernel whose name contains
KERNEL_SUBSTR: each counter (KiB per dispatch) is scaled by the factor that
maps the same counter of a plain device copy of COPY_BYTES bytes (the largest
copy kernel in the run, which reads and writes COPY_BYTES each) onto its known
size, over all its dispatches or its last LAST_N (CSV input).  ``tail`` splits the dispatches of the kernel whose name contains
KERNEL_SUBSTR, in start order, into all but the last N and the last N, and
prints count and average duration of each part and the median start-to-start
period of the last N (a timed graph replay is the last dispatches of a run).
``phases`` sorts the last REPS x R x L dispatches of that kernel (REPS timed
replays of a graph of whole merge cycles over R pools decoded in turn, pool
t mod R at step t, every slot of a pool in the same phase) by the live-log
length n each one started from: within a replay, every R-th dispatch belongs
to one pool, its longest dispatch is that pool's merge (n = L - 1), and the
dispatch k places after it starts from n = k - 1.  Prints the average duration
per n.
Works on the SQLite database rocprofv3 writes by default (``*_results.db``)
and on its CSV output (``tail``: CSV only).
"""

from __future__ import annotations

import csv
import os
import sqlite3
import sys
from collections import defaultdict


def _short(name: str, width: int = 100) -> str:
    return name if len(name) <= width else name[: width - 3] + "..."


def trace_rows(path: str):
    """[(name, count, avg_ns, min_ns, max_ns, total_ns)] sorted by total time."""
    agg = defaultdict(list)
    if path.endswith(".db"):
        con = sqlite3.connect(path)
        for name, dur in con.execute("select name, duration from kernels"):
            agg[name].append(float(dur))
    else:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name") or r.get("KernelName") or r.get("Name")
                if "Start_Timestamp" in r:
                    agg[name].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
                elif "AverageNs" in r:
                    agg[name].extend([float(r["AverageNs"])] * int(r["Calls"]))
    rows = [(n, len(v), sum(v) / len(v), min(v), max(v), sum(v)) for n, v in agg.items()]
    return sorted(rows, key=lambda r: -r[5])


def trace_tail(path: str, sub: str, n: int):
    """(count_head, avg_head_ns, count_tail, avg_tail_ns, median_period_tail_ns) of
    one kernel's dispatches in start order, the tail being the last n."""
    spans = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if sub in (r.get("Kernel_Name") or ""):
                spans.append((float(r["Start_Timestamp"]), float(r["End_Timestamp"])))
    spans.sort()
    head, tail = spans[:-n] if n < len(spans) else [], spans[-n:]
    avg = lambda xs: sum(e - s for s, e in xs) / len(xs) if xs else 0.0
    starts = [s for s, _ in tail]
    per = sorted(b - a for a, b in zip(starts, starts[1:]))
    return len(head), avg(head), len(tail), avg(tail), (per[len(per) // 2] if per else 0.0)


def trace_phases(path: str, sub: str, R: int, L: int, reps: int):
    """{n: [duration ns]} of the last reps * R * L dispatches of one kernel."""
    spans = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if sub in (r.get("Kernel_Name") or ""):
                spans.append((float(r["Start_Timestamp"]), float(r["End_Timestamp"])))
    spans.sort()
    per = R * L
    spans = spans[-reps * per:]
    by = defaultdict(list)
    for rep in range(len(spans) // per):
        blk = spans[rep * per:(rep + 1) * per]
        for p in range(R):
            durs = [e - s for s, e in blk[p::R]]
            km = max(range(len(durs)), key=lambda k: durs[k])
            for k, dur in enumerate(durs):
                by[L - 1 if k == km else (k - km - 1) % L].append(dur)
    return by


def pmc_dispatches(path: str, counter: str):
    """{kernel name: [value of COUNTER per dispatch]}."""
    per = defaultdict(lambda: defaultdict(float))
    if path.endswith(".db"):
        con = sqlite3.connect(path)
        rows = con.execute("select kernel_name, dispatch_id, counter_value from counters_collection "
                           "where counter_name = ?", (counter,)).fetchall()
        for name, did, val in rows:
            per[name][did] += float(val)
    else:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {n: list(d.values()) for n, d in per.items()}


def _pmc_by_dispatch(path: str, counter: str):
    """{kernel name: {dispatch id: value of COUNTER}} (CSV output)."""
    per = defaultdict(lambda: defaultdict(float))
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return per


def pmc_rows(path: str, counter: str):
    """[(name, dispatches, avg value per dispatch)]."""
    per = defaultdict(lambda: defaultdict(float))     # name -> dispatch -> value
    if path.endswith(".db"):
        con = sqlite3.connect(path)
        q = ("select k.name, p.dispatch_id, p.value from pmc_events p join kernels k "
             "on p.dispatch_id = k.dispatch_id where p.counter_name = ?")
        try:
            rows = con.execute(q, (counter,)).fetchall()
        except sqlite3.OperationalError:
            rows = con.execute("select kernel_name, dispatch_id, counter_value from counters_collection "
                               "where counter_name = ?", (counter,)).fetchall()
        for name, did, val in rows:
            per[name][did] += float(val)
    else:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    out = []
    for name, d in per.items():
        vals = list(d.values())
        out.append((name, len(vals), sum(vals) / len(vals)))
    return sorted(out, key=lambda r: -r[2] * r[1])


CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def kernel_source_hash() -> str:
    """Hash of the HIP sources: counters taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(fetch_path: str, write_path: str, kernel: str, copy_bytes: int, last: int = 0) -> dict:
    """HBM bytes per launch of the kernel matching `kernel` (most dispatches),
    averaged over all its dispatches or, with last > 0, over its last `last`
    dispatches (the timed steps, after set-up and warm-up launches)."""

    def rows_of(path, counter):
        # (name, dispatches in the run, dispatches averaged, average)
        if not last:
            return [(n, k, k, v) for n, k, v in pmc_rows(path, counter)]
        out = []
        for name, did_vals in _pmc_by_dispatch(path, counter).items():
            ids = sorted(did_vals, key=lambda x: int(x))
            v = [did_vals[i] for i in ids[-last:]]
            out.append((name, len(ids), len(v), sum(v) / len(v)))
        return out

    f_rows = rows_of(fetch_path, "FETCH_SIZE")
    w_rows = rows_of(write_path, "WRITE_SIZE")

    def pick(rows, sub):
        m = [r for r in rows if sub in r[0]]
        if not m:
            raise SystemExit(f"no kernel matching {sub!r}")
        # most dispatches in the whole run (with `last`, every kernel that ran
        # at least `last` times averages the same number of them)
        return max(m, key=lambda r: r[1])

    def copy_row(path, counter):
        # the single largest dispatch of a copy kernel: the calibration copy
        best = None
        for name, vals in pmc_dispatches(path, counter).items():
            if "copy" in name.lower():
                v = max(vals)
                if best is None or v > best[2]:
                    best = (name, 1, v)
        return best

    kf = pick(f_rows, kernel)
    kw = next((r for r in w_rows if r[0] == kf[0]), None) or pick(w_rows, kernel)
    cf, cw = copy_row(fetch_path, "FETCH_SIZE"), copy_row(write_path, "WRITE_SIZE")
    f_scale = copy_bytes / (cf[2] * 1024.0) if cf else 1.0
    w_scale = copy_bytes / (cw[2] * 1024.0) if cw else 1.0
    fetch_b = kf[3] * 1024.0 * f_scale
    write_b = kw[3] * 1024.0 * w_scale
    return {"kernel": kf[0], "dispatches": kf[2], "fetch_kib_per_dispatch": kf[3],
            "write_kib_per_dispatch": kw[3], "copy_kernel": cf[0] if cf else None,
            "copy_fetch_kib": cf[2] if cf else None, "copy_write_kib": cw[2] if cw else None,
            "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
            "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
            "hbm_bytes_per_launch": fetch_b + write_b, "kernel_source_hash": kernel_source_hash()}


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) < 2:
        print(__doc__)
        return 2
    mode, path = argv[0], argv[1]
    print(f"# source: {os.path.basename(path)}")
    if mode == "trace":
        print(f"{'kernel':100s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
        for n, c, a, lo, hi, _ in trace_rows(path):
            print(f"{_short(n):100s} {c:6d} {a / 1e3:9.3f} {lo / 1e3:9.3f} {hi / 1e3:9.3f}")
    elif mode == "pmc":
        counter = argv[2]
        print(f"{'kernel':100s} {'dispatches':>10s} {counter + '/dispatch':>20s}")
        for n, c, v in pmc_rows(path, counter):
            print(f"{_short(n):100s} {c:10d} {v:20.1f}")
    elif mode == "tail":
        nh, ah, nt, at, pt = trace_tail(path, argv[2], int(argv[3]))
        print(f"kernel containing: {argv[2]}")
        print(f"first {nh} dispatches: avg {ah / 1e3:.3f} us")
        print(f"last {nt} dispatches: avg {at / 1e3:.3f} us, median start-to-start {pt / 1e3:.3f} us")
    elif mode == "phases":
        by = trace_phases(path, argv[2], int(argv[3]), int(argv[4]), int(argv[5]))
        print(f"kernel containing: {argv[2]}")
        print(f"{'n':>3s} {'dispatches':>10s} {'avg_us':>9s}")
        for n in sorted(by):
            print(f"{n:3d} {len(by[n]):10d} {sum(by[n]) / len(by[n]) / 1e3:9.3f}")
    elif mode == "traffic":
        import json
        last = int(argv[6]) if len(argv) > 6 else 0
        t = traffic(argv[1], argv[2], argv[3], int(argv[4]), last)
        t["dispatches_averaged"] = "last %d" % last if last else "all"
        txt = json.dumps(t, indent=1)
        print(txt)
        if len(argv) > 5 and argv[5] != "-":
            with open(argv[5], "w") as f:
                f.write(txt + "\n")
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main())
