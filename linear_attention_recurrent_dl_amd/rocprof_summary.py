"""Summarize rocprofv3 output (kernel trace and PMC counters) as short text.

    python -m linear_attention_recurrent_dl_amd.rocprof_summary trace  <results.db | kernel_trace.csv>
    python -m linear_attention_recurrent_dl_amd.rocprof_summary pmc    <results.db | counter_collection.csv> COUNTER

``trace`` prints count / average / min / max duration per kernel name;
``pmc`` prints, per kernel name, the average value of COUNTER per dispatch and
the number of dispatches.  Works on the SQLite database rocprofv3 writes by
default (``*_results.db``) and on its CSV output.
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
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main())
