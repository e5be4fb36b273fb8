"""Summaries of rocprofv3 results databases, for the text files kept under profiles/.

    python -m rag_kv_cache_amd.profsummary trace <results.db> [--steps L,FIRST,COUNT]
        [--role LABEL=REGEX ...] [--command ...] [--out file]
        per kernel symbol: launches, total / average / min / max duration; then, with --steps,
        per kernel the launches and average duration over steps FIRST .. FIRST+COUNT-1 (a step
        starts at its embedding launch), and per --role the average over those steps' launches
        whose kernel name matches REGEX
    python -m rag_kv_cache_amd.profsummary traffic <fetch.db> <write.db> --kernel REGEX
        [--calib-grid N --calib-bytes B] [--source FILE] [--command ...] [--out file]
        FETCH_SIZE / WRITE_SIZE per dispatch of the kernels matching REGEX, grouped by grid
        size, each scaled by what the counter reads for a plain device copy of B bytes (the
        dispatch with grid N); the sha256 of FILE is recorded so that a reader can tell
        whether the kernel source changed since the counters were taken; with --last N, also
        the average over the last N matching dispatches (one step's launches when the profiled
        run ends with a step)
    python -m rag_kv_cache_amd.profsummary counters <results.db> [<results.db> ...] --kernel REGEX
        [--cus 256] [--last N]
        every counter of the matching dispatches, mean per (kernel, grid), from one or more
        counter runs (one pass per run); derived where the inputs are there: MFMA busy share
        SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x CUs x 4 SIMDs), VALU instructions per
        MFMA instruction, LDS-wait share of wave cycles; --last N also averages the last N
        matching dispatches
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


def step_kernels(db_path: str, n_layers: int, first_step: int, n_steps: int, roles=()) -> str:
    """Per-kernel averages over steps first_step .. first_step+n_steps-1 of a run whose steps each
    hold exactly n_layers embed-delimited layers; a step starts at an embedding launch.  roles:
    (label, regex) pairs; each gets the average over every launch in those steps whose kernel
    name matches (e.g. one product's launches at every layer, whatever the instantiation)."""
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
    for label, rx in roles:
        v = [dur for name, dur, _, _, _ in rows[lo:hi] if re.search(rx, _short(name))]
        if v:
            lines.append(f"role {label}: {len(v) / n_steps:.1f} launches per step, {statistics.mean(v) / 1e3:.2f} us "
                         f"per launch on average, {sum(v) / 1e3 / n_steps:.2f} us per step (kernels matching {rx!r})")
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
    cf = [statistics.mean(v) for (n, g), v in f.items() if g == calib_grid and "copyBuffer" in n]
    cw = [statistics.mean(v) for (n, g), v in w.items() if g == calib_grid and "copyBuffer" in n]
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


def _dispatch_counters(path: str, kernel_re: str):
    """{dispatch_id: (kernel name, grid, {counter: value})} of the matching dispatches."""
    db = sqlite3.connect(path)
    rx = re.compile(kernel_re)
    out = {}
    for did, name, cn, val, gs in db.execute(
            "select dispatch_id, kernel_name, counter_name, value, grid_size from counters_collection"):
        if not rx.search(name):
            continue
        rec = out.setdefault(did, (name, gs, {}))
        rec[2][cn] = rec[2].get(cn, 0.0) + val
    return out


def counters(paths, kernel_re: str, cus: int, last: int, xcds: int = 8, label: str = "") -> str:
    runs = [_dispatch_counters(p, kernel_re) for p in paths]
    groups = defaultdict(lambda: defaultdict(list))
    for run in runs:
        for did in sorted(run):
            name, gs, vals = run[did]
            for cn, v in vals.items():
                groups[(_short(name).split("(")[0], gs)][cn].append(v)
    names = sorted({cn for g in groups.values() for cn in g})
    lines = [f"{'grid':>9} {'n':>5} " + " ".join(f"{n[:22]:>22}" for n in names) + "  derived  kernel"]

    def derived(m):
        parts = []
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and m.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE is summed over the XCDs: one XCD's count is the dispatch's cycles
            cyc = m["GRBM_GUI_ACTIVE"] / xcds
            parts.append(f"mfma_busy {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * cus * 4):.3f}")
        if "SQ_INSTS_VALU" in m and m.get("SQ_INSTS_MFMA"):
            parts.append(f"valu/mfma {m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f}")
        if "SQ_WAIT_INST_LDS" in m and m.get("SQ_WAVE_CYCLES"):
            parts.append(f"lds_wait/wave {m['SQ_WAIT_INST_LDS'] / m['SQ_WAVE_CYCLES']:.3f}")
        if "SQ_ACTIVE_INST_VALU" in m and m.get("SQ_WAVE_CYCLES"):
            parts.append(f"valu_active/wave {m['SQ_ACTIVE_INST_VALU'] / m['SQ_WAVE_CYCLES']:.3f}")
        return ", ".join(parts)

    for (name, gs), cmap in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        m = {cn: statistics.mean(v) for cn, v in cmap.items()}
        n = max(len(v) for v in cmap.values())
        lines.append(f"{gs:9d} {n:5d} " + " ".join(f"{m.get(c, float('nan')):22.0f}" for c in names)
                     + f"  {derived(m)}  {name[:70]}")
    if last:
        m = {}
        for run in runs:
            dids = sorted(run)[-last:]
            for cn in {c for d in dids for c in run[d][2]}:
                m[cn] = statistics.mean(run[d][2].get(cn, 0.0) for d in dids)
        lines.append((f"{label}: " if label else "") + f"last {last} dispatches: "
                     + ", ".join(f"{c} {m[c]:.0f}" for c in sorted(m)) + (f"; {derived(m)}" if derived(m) else ""))
    return "\n".join(lines)


def traffic_last(fetch_db: str, write_db: str, kernel_re: str, calib_grid: int, calib_bytes: float, last: int) -> str:
    """Mean scaled HBM bytes of the last `last` matching dispatches (in dispatch order)."""
    f = _dispatch_counters(fetch_db, kernel_re + "|copyBuffer")
    w = _dispatch_counters(write_db, kernel_re + "|copyBuffer")
    kib = calib_bytes / 1024.0
    cf = [v[2]["FETCH_SIZE"] for v in f.values() if v[1] == calib_grid and "copyBuffer" in v[0]]
    cw = [v[2]["WRITE_SIZE"] for v in w.values() if v[1] == calib_grid and "copyBuffer" in v[0]]
    sf = kib / statistics.mean(cf) if cf else float("nan")
    sw = kib / statistics.mean(cw) if cw else float("nan")
    rx = re.compile(kernel_re)
    fd = [d for d in sorted(f) if rx.search(f[d][0])][-last:]
    wd = [d for d in sorted(w) if rx.search(w[d][0])][-last:]
    if len(fd) < last or len(wd) < last:
        return f"(fewer than {last} matching dispatches)"
    mb = statistics.mean(f[d][2]["FETCH_SIZE"] * sf for d in fd) * 1024 / 1e6 + \
        statistics.mean(w[d][2]["WRITE_SIZE"] * sw for d in wd) * 1024 / 1e6
    return f"step average over the last {last} launches: {mb:.2f} MB per launch"


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--steps", default="", help="N_LAYERS,FIRST,COUNT: per-step kernel averages")
    t.add_argument("--role", action="append", default=[], help="LABEL=REGEX: average over a step's matching launches")
    x = sub.add_parser("traffic")
    x.add_argument("fetch_db")
    x.add_argument("write_db")
    x.add_argument("--kernel", required=True)
    x.add_argument("--calib-grid", type=int, default=131072)
    x.add_argument("--calib-bytes", type=float, default=float(256 << 20))
    x.add_argument("--source", action="append", default=[])
    x.add_argument("--last", type=int, default=0)
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--last", type=int, default=0)
    c.add_argument("--label", default="", help="name printed before the --last line")
    c.add_argument("--only-last", action="store_true", help="print only the --last line")
    for p in (t, x, c):
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
            roles = [tuple(r.split("=", 1)) for r in a.role]
            text += "\n" + step_kernels(a.db, nl, first, cnt, roles) + "\n"
    elif a.cmd == "counters":
        out = counters(a.dbs, a.kernel, a.cus, a.last, a.xcds, a.label)
        text += (out.splitlines()[-1] if a.only_last else out) + "\n"
    else:
        for src in a.source:
            text += f"source_sha256 {src}: {hashlib.sha256(open(src, 'rb').read()).hexdigest()}\n"
        text += traffic(a.fetch_db, a.write_db, a.kernel, a.calib_grid, a.calib_bytes) + "\n"
        if a.last:
            text += traffic_last(a.fetch_db, a.write_db, a.kernel, a.calib_grid, a.calib_bytes, a.last) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    else:
        sys.stdout.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
