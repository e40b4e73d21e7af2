"""Summaries of rocprofv3 output databases (kernel durations, PMC counters).

    python -m progressive_kv_transfer_amd.profiling trace RESULTS_DB [--match lynx]
    python -m progressive_kv_transfer_amd.profiling pmc RESULTS_DB [--match lynx]
    python -m progressive_kv_transfer_amd.profiling traffic FETCH_DB WRITE_DB \
        COPY_FETCH_DB COPY_WRITE_DB --elements N [--title T]
    python -m progressive_kv_transfer_amd.profiling copies RESULTS_DB

`trace` prints, per kernel, the number of dispatches and the average,
minimum and maximum duration (from the kernel-trace table); `pmc` prints, per
kernel and counter (rocprofv3 --pmc), the per-dispatch value averaged over
the dispatches; `traffic` turns FETCH_SIZE / WRITE_SIZE passes over the codec
kernels (and over a plain 1 GiB copy, which fixes the counters' scale) into
HBM bytes per launch against the algorithmic bytes of N bf16 elements, as a
markdown table plus the JSON block that bench.py reads; `copies` summarises
the host <-> device copies of a --memory-copy-trace run and the runtime's
shader blit copies.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sqlite3
import statistics

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# Sources of the codec kernels whose traffic the committed summary describes.
CODEC_SOURCES = ("lynx_quant.hip", "lynx_dequant.hip", "lynx_recon.h", "lynx_internal.h",
                 "lynx_device.h")
# kernel symbol -> (name, algorithmic HBM bytes per bf16 element)
CODEC_KERNELS = {
    "lynx::quant_kernel<0, true, 4, 4, false>": ("quantize", 2.0 + 0.5 + 0.5 + 0.28125),
    "lynx::quant_kernel<0, false, 4, 4, false>": ("quantize", 2.0 + 0.5 + 0.5 + 0.28125),
    "lynx::dequant_kernel<false, 4, 4, false>": ("dequant_anchor", 0.5 + 0.28125 + 2.0),
    "lynx::dequant_kernel<true, 4, 4, false>": ("dequant_full", 0.5 + 0.5 + 0.28125 + 2.0),
}
COPY_BYTES = 1 << 30


def kernel_source_hash(files=CODEC_SOURCES) -> str:
    """SHA-256 prefix of the kernel sources (a summary taken on other
    sources no longer describes the kernels)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def _counter(db: str, match: str, counter: str) -> dict:
    return {k: vsum for k, c, _, vsum, _ in pmc(db, match) if c == counter}


def traffic(fetch_db, write_db, copy_fetch_db, copy_write_db, elements: int,
            title: str, command: str) -> str:
    cf = list(_counter(copy_fetch_db, "copy", "FETCH_SIZE").values())[0]
    cw = list(_counter(copy_write_db, "copy", "WRITE_SIZE").values())[0]
    fscale = COPY_BYTES / 1024.0 / cf
    wscale = COPY_BYTES / 1024.0 / cw
    fetch = _counter(fetch_db, "lynx", "FETCH_SIZE")
    write = _counter(write_db, "lynx", "WRITE_SIZE")
    gib = float(1 << 30)
    rows, kern = [], {}
    for sym, (name, bpe) in CODEC_KERNELS.items():
        if sym not in fetch or sym not in write:
            continue
        rd = fetch[sym] * 1024.0 * fscale
        wr = write[sym] * 1024.0 * wscale
        algo = bpe * elements
        rows.append(f"| {sym} | {fetch[sym]:.0f} | {write[sym]:.0f} | {rd / gib:.4f} GiB | "
                    f"{wr / gib:.4f} GiB | {(rd + wr) / gib:.4f} GiB | {algo / gib:.4f} GiB | "
                    f"{(rd + wr) / algo:.4f} |")
        kern[name] = {"kernel": sym, "fetch_size_kib": round(fetch[sym], 1),
                      "write_size_kib": round(write[sym], 1), "hbm_read_bytes": int(rd),
                      "hbm_write_bytes": int(wr), "hbm_bytes_per_launch": int(rd + wr),
                      "algorithmic_bytes_per_launch": int(algo)}
    blob = {"kernel_source_hash": kernel_source_hash(), "fetch_scale": fscale,
            "write_scale": wscale,
            "copy_probe": {"bytes": COPY_BYTES, "fetch_size_kib": cf, "write_size_kib": cw},
            "kernels": kern}
    out = [f"# HBM traffic per launch: {title}", "",
           "Commands (on an MI355X, repository root `$R`, one counter per pass):", "",
           *("    " + line for line in command.strip().splitlines()), "",
           f"Scale factors from a plain 1 GiB device copy (`bench.py --copy-probe`): "
           f"FETCH_SIZE reads {cf:.0f} KiB for 1 GiB fetched (x{fscale:.3f}); WRITE_SIZE "
           f"reads {cw:.0f} KiB for 1 GiB written (x{wscale:.3f}).", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read (scaled) | HBM write | total "
           "| algorithmic | ratio |", "|---|---|---|---|---|---|---|---|", *rows, "",
           "Machine-readable (read by bench.py; `kernel_source_hash` is the SHA-256 prefix of "
           "the kernel sources the counters were taken on):", "", "```json",
           json.dumps(blob, indent=1), "```"]
    return "\n".join(out) + "\n"


TRAFFIC_COMMAND = """
cd /tmp && export TMPDIR=/tmp
rocprofv3 --pmc FETCH_SIZE -d /tmp/pr/FETCH_SIZE -o run -- python3 $R/bench.py --profile-run
rocprofv3 --pmc WRITE_SIZE -d /tmp/pr/WRITE_SIZE -o run -- python3 $R/bench.py --profile-run
rocprofv3 --pmc FETCH_SIZE -d /tmp/pr/copy_FETCH_SIZE -o run -- python3 $R/bench.py --copy-probe
rocprofv3 --pmc WRITE_SIZE -d /tmp/pr/copy_WRITE_SIZE -o run -- python3 $R/bench.py --copy-probe
cd $R && python3 -m progressive_kv_transfer_amd.profiling traffic \\
    /tmp/pr/FETCH_SIZE/run_results.db /tmp/pr/WRITE_SIZE/run_results.db \\
    /tmp/pr/copy_FETCH_SIZE/run_results.db /tmp/pr/copy_WRITE_SIZE/run_results.db \\
    --elements 2147483648
"""


def copies(db: str):
    """Host <-> device copies of a --memory-copy-trace run, by direction and
    size (>= 32 MiB = big), and the runtime's shader blit copies
    (`__amd_rocclr_copyBuffer` dispatches) by duration."""
    c = sqlite3.connect(db)
    names = [r[0] for r in c.execute("select name from sqlite_master")]
    agents = (dict(c.execute("select id, type from rocpd_info_agent").fetchall())
              if "rocpd_info_agent" in names else {})
    groups = {}
    for src, dst, size, dur in c.execute(
            "select src_agent_id, dst_agent_id, size, end - start from rocpd_memory_copy"):
        k = (agents.get(src, src), agents.get(dst, dst), "big" if size >= 32 << 20 else "small")
        g = groups.setdefault(k, [0, 0, 0])
        g[0] += 1
        g[1] += size
        g[2] += dur
    blits = [d for (d,) in c.execute(
        "select k.end - k.start from rocpd_kernel_dispatch k join rocpd_info_kernel_symbol s "
        "on k.kernel_id = s.id where s.kernel_name like '%copyBuffer%'")]
    return groups, blits


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc", "traffic", "copies"])
    ap.add_argument("db", nargs="+")
    ap.add_argument("--match", default=None)
    ap.add_argument("--elements", type=int, default=1 << 31)
    ap.add_argument("--title", default="Qwen-32B-shaped KV at 16K (64 layers x K,V x 16384 x "
                                        "1024 bf16)")
    a = ap.parse_args()
    if a.mode == "traffic":
        if len(a.db) != 4:
            ap.error("traffic needs FETCH_DB WRITE_DB COPY_FETCH_DB COPY_WRITE_DB")
        print(traffic(*a.db, a.elements, a.title, TRAFFIC_COMMAND), end="")
        return
    a.db = a.db[0]
    if a.mode == "copies":
        groups, blits = copies(a.db)
        print("| from | to | size | copies | GB | avg us | GB/s while copying |")
        print("|---|---|---|---|---|---|---|")
        for (src, dst, cls), (n, b, t) in sorted(groups.items(), key=str):
            print(f"| {src} | {dst} | {cls} | {n} | {b / 1e9:.2f} | {t / n / 1e3:.1f} | "
                  f"{b / t if t else 0.0:.1f} |")
        print()
        print("| shader blit copies | dispatches | under 100 us | 100 us - 1 ms | over 1 ms |")
        print("|---|---|---|---|---|")
        print(f"| __amd_rocclr_copyBuffer | {len(blits)} | {sum(d <= 1e5 for d in blits)} | "
              f"{sum(1e5 < d <= 1e6 for d in blits)} | {sum(d > 1e6 for d in blits)} |")
        return
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
