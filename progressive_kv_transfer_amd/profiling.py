"""Summaries of rocprofv3 output databases (kernel durations, PMC counters).

    python -m progressive_kv_transfer_amd.profiling trace RESULTS_DB [--match lynx]
    python -m progressive_kv_transfer_amd.profiling pmc RESULTS_DB COUNTER [--match lynx]

`trace` prints, per kernel, the number of dispatches and the average,
minimum and maximum duration (from the kernel-trace table); `pmc` prints the
per-dispatch value of one counter (rocprofv3 --pmc), averaged per kernel.
"""
from __future__ import annotations

import argparse
import sqlite3
import statistics


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0]


def trace(db: str, match: str | None = None):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    by = {}
    for name, dur in rows:
        if match and match not in name:
            continue
        by.setdefault(_short(name), []).append(dur / 1e3)  # ns -> us
    out = []
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append((k, len(v), statistics.mean(v), min(v), max(v)))
    return out


def pmc(db: str, counter: str, match: str | None = None):
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(pmc_events)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    val_col = "counter_value" if "counter_value" in cols else "value"
    cnt_col = "counter_name" if "counter_name" in cols else "pmc_name"
    disp_col = "dispatch_id" if "dispatch_id" in cols else "id"
    rows = con.execute(
        f"select {name_col}, {disp_col}, sum({val_col}) from pmc_events "
        f"where {cnt_col} = ? group by {name_col}, {disp_col}", (counter,)).fetchall()
    by = {}
    for name, _, v in rows:
        if match and match not in name:
            continue
        by.setdefault(_short(name), []).append(v)
    return [(k, len(v), statistics.mean(v)) for k, v in sorted(by.items())]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc"])
    ap.add_argument("db")
    ap.add_argument("counter", nargs="?")
    ap.add_argument("--match", default=None)
    a = ap.parse_args()
    if a.mode == "trace":
        print("| kernel | dispatches | avg us | min us | max us |")
        print("|---|---|---|---|---|")
        for k, n, avg, mn, mx in trace(a.db, a.match):
            print(f"| {k} | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")
    else:
        print(f"| kernel | dispatches | avg {a.counter} per dispatch |")
        print("|---|---|---|")
        for k, n, avg in pmc(a.db, a.counter, a.match):
            print(f"| {k} | {n} | {avg:.1f} |")


if __name__ == "__main__":
    main()
