"""Summaries of rocprofv3 output databases (kernel durations, PMC counters).

    python -m progressive_kv_transfer_amd.profiling trace RESULTS_DB [--match lynx]
    python -m progressive_kv_transfer_amd.profiling pmc RESULTS_DB [--match lynx]

`trace` prints, per kernel, the number of dispatches and the average,
minimum and maximum duration (from the kernel-trace table); `pmc` prints, per
kernel and counter (rocprofv3 --pmc), the per-dispatch value averaged over
the dispatches.
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


def pmc(db: str, match: str | None = None):
    """Per kernel and counter: number of dispatches and the per-dispatch
    average of the counter summed over its hardware instances (and of the
    per-instance maximum, the right reduction for GRBM_GUI_ACTIVE)."""
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, dispatch_id, counter_name, sum(counter_value), max(counter_value) "
        "from pmc_events group by dispatch_id, counter_name").fetchall()
    by = {}
    for name, _, cname, vsum, vmax in rows:
        if match and match not in name:
            continue
        by.setdefault((_short(name), cname), []).append((vsum, vmax))
    return [(k, c, len(v), statistics.mean(x[0] for x in v), statistics.mean(x[1] for x in v))
            for (k, c), v in sorted(by.items())]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc"])
    ap.add_argument("db")
    ap.add_argument("--match", default=None)
    a = ap.parse_args()
    if a.mode == "trace":
        print("| kernel | dispatches | avg us | min us | max us |")
        print("|---|---|---|---|---|")
        for k, n, avg, mn, mx in trace(a.db, a.match):
            print(f"| {k} | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")
    else:
        print("| kernel | counter | dispatches | avg sum over instances | avg max instance |")
        print("|---|---|---|---|---|")
        for k, c, n, vsum, vmax in pmc(a.db, a.match):
            print(f"| {k} | {c} | {n} | {vsum:.1f} | {vmax:.1f} |")


if __name__ == "__main__":
    main()
