"""Summarise a rocprofv3 results database (kernel trace) into a short text table.

    python -m rag_kv_cache_amd.profsummary <results.db> [--command "..."] [--out file]

Per kernel symbol: launches, total / average / min / max duration.  Used to write the
summaries committed under profiles/.
"""
from __future__ import annotations

import argparse
import sqlite3
import statistics
import sys
from collections import defaultdict


def summarise(db_path: str) -> str:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, duration, grid_x, grid_y, workgroup_x from kernels").fetchall()
    agg = defaultdict(list)
    for name, dur, gx, gy, wx in rows:
        agg[name].append(dur)
    total = sum(sum(v) for v in agg.values())
    lines = [f"{'launches':>8} {'total_ms':>10} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}  kernel"]
    for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v):8d} {sum(v) / 1e6:10.3f} {statistics.mean(v) / 1e3:9.2f} {min(v) / 1e3:9.2f} "
                     f"{max(v) / 1e3:9.2f} {100.0 * sum(v) / total:6.2f}  {name[:150]}")
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--command", default="")
    ap.add_argument("--note", default="")
    ap.add_argument("--out", default="")
    a = ap.parse_args()
    text = ""
    if a.command:
        text += f"command: {a.command}\n"
    if a.note:
        text += a.note + "\n"
    text += summarise(a.db) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    else:
        sys.stdout.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
