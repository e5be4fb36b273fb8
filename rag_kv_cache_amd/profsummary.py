"""Summaries of rocprofv3 results databases, for the text files kept under profiles/.

    python -m rag_kv_cache_amd.profsummary trace <results.db> [--command ...] [--out file]
        per kernel symbol: launches, total / average / min / max duration; then, for the
        kernels of one blended-prefill step (identified by their grid sizes), the average
        duration per launch over the steps replayed from the HIP graph
    python -m rag_kv_cache_amd.profsummary traffic <fetch.db> <write.db> --kernel REGEX
        [--calib-grid N --calib-bytes B] [--source FILE] [--command ...] [--out file]
        FETCH_SIZE / WRITE_SIZE per dispatch of the kernels matching REGEX, grouped by grid
        size, each scaled by what the counter reads for a plain device copy of B bytes (the
        dispatch with grid N); the sha256 of FILE is recorded so that a reader can tell
        whether the kernel source changed since the counters were taken
"""
from __future__ import annotations

import argparse
import hashlib
import re
import sqlite3
import statistics
import sys
from collections import defaultdict


def _short(name: str) -> str:
    return name.replace("void cb::(anonymous namespace)::", "").replace("cb::(anonymous namespace)::", "")


def trace_table(db_path: str) -> str:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, duration from kernels").fetchall()
    agg = defaultdict(list)
    for name, dur in rows:
        agg[name].append(dur)
    total = sum(sum(v) for v in agg.values())
    lines = [f"{'launches':>8} {'total_ms':>10} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}  kernel"]
    for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v):8d} {sum(v) / 1e6:10.3f} {statistics.mean(v) / 1e3:9.2f} {min(v) / 1e3:9.2f} "
                     f"{max(v) / 1e3:9.2f} {100.0 * sum(v) / total:6.2f}  {_short(name)[:140]}")
    return "\n".join(lines)


def step_kernels(db_path: str, n_layers: int, first_step: int, n_steps: int) -> str:
    """Per-kernel averages over steps first_step .. first_step+n_steps-1 of a run whose steps each
    hold exactly n_layers embed-delimited layers; a step starts at an embedding launch."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, duration, grid_x, grid_y, start from kernels order by start").fetchall()
    starts = [i for i, r in enumerate(rows) if "embed_kernel" in r[0]]
    if len(starts) < first_step + n_steps + 1:
        return "(not enough steps in the trace)"
    lo, hi = starts[first_step], starts[first_step + n_steps]
    agg = defaultdict(list)
    for name, dur, gx, gy, _ in rows[lo:hi]:
        agg[_short(name).split("(")[0]].append(dur)
    span = (rows[hi][4] - rows[lo][4]) / 1e3 / n_steps
    lines = [f"steps {first_step}..{first_step + n_steps - 1}: {span:.1f} us per step (first launch to next step's first)",
             f"{'per_step':>8} {'us_per_step':>11} {'avg_us':>9}  kernel"]
    for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v) / n_steps:8.1f} {sum(v) / 1e3 / n_steps:11.2f} {statistics.mean(v) / 1e3:9.2f}  {name[:100]}")
    return "\n".join(lines)


def traffic(fetch_db: str, write_db: str, kernel_re: str, calib_grid: int, calib_bytes: float) -> str:
    def read(path, counter):
        db = sqlite3.connect(path)
        agg = defaultdict(list)
        for name, cn, val, gs in db.execute("select kernel_name, counter_name, value, grid_size from counters_collection"):
            if cn == counter:
                agg[(name, gs)].append(val)
        return agg
    f, w = read(fetch_db, "FETCH_SIZE"), read(write_db, "WRITE_SIZE")
    cf = [statistics.mean(v) for (n, g), v in f.items() if g == calib_grid]
    cw = [statistics.mean(v) for (n, g), v in w.items() if g == calib_grid]
    kib = calib_bytes / 1024.0
    sf = kib / cf[0] if cf else float("nan")
    sw = kib / cw[0] if cw else float("nan")
    lines = [f"calibration: plain device copy of {calib_bytes / 2**20:.0f} MiB read + written (grid {calib_grid}): "
             f"FETCH_SIZE {cf[0] if cf else float('nan'):.1f} KiB -> factor {sf:.4f}; "
             f"WRITE_SIZE {cw[0] if cw else float('nan'):.1f} KiB -> factor {sw:.4f}",
             f"{'grid':>8} {'launches':>8} {'fetch_KiB':>11} {'write_KiB':>11} {'scaled_MB':>10}  kernel"]
    rx = re.compile(kernel_re)
    for (name, g), v in sorted(f.items(), key=lambda kv: kv[0][1]):
        if not rx.search(name):
            continue
        fk = statistics.mean(v)
        wk = statistics.mean(w.get((name, g), [float("nan")]))
        mb = (fk * sf + wk * sw) * 1024 / 1e6
        lines.append(f"{g:8d} {len(v):8d} {fk:11.1f} {wk:11.1f} {mb:10.2f}  {_short(name)[:90]}")
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--steps", default="", help="N_LAYERS,FIRST,COUNT: per-step kernel averages")
    x = sub.add_parser("traffic")
    x.add_argument("fetch_db")
    x.add_argument("write_db")
    x.add_argument("--kernel", required=True)
    x.add_argument("--calib-grid", type=int, default=131072)
    x.add_argument("--calib-bytes", type=float, default=float(256 << 20))
    x.add_argument("--source", default="")
    for p in (t, x):
        p.add_argument("--command", action="append", default=[])
        p.add_argument("--note", default="")
        p.add_argument("--out", default="")
    a = ap.parse_args()
    text = "".join(f"command: {c}\n" for c in a.command)
    if a.note:
        text += a.note + "\n"
    if a.cmd == "trace":
        text += trace_table(a.db) + "\n"
        if a.steps:
            nl, first, cnt = (int(v) for v in a.steps.split(","))
            text += "\n" + step_kernels(a.db, nl, first, cnt) + "\n"
    else:
        if a.source:
            text += f"source_sha256 {a.source}: {hashlib.sha256(open(a.source, 'rb').read()).hexdigest()}\n"
        text += traffic(a.fetch_db, a.write_db, a.kernel, a.calib_grid, a.calib_bytes) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    else:
        sys.stdout.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
