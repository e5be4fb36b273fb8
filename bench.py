#!/usr/bin/env python3
"""Benchmark of the blended (CacheBlend-fused) prefill on one MI355X.

One step = one whole blended prefill of the Llama-70B-shaped workload at 16K context: 80
decoder layers, d_model 8192, 64 query / 8 KV heads of 128, FFN 28672, bf16, random-init
weights N(0, 0.02) (about 137 GB, drawn on the device); 32 independently cached chunks of 512
uniform-random tokens + a 256-token query; layer 1 recomputes every row, layers 2.. keep 15% of
the context rows.  The chunks' cached K/V sit in pinned host memory (the library's chunk store,
filled by the chunk producer) and are fetched per layer over PCIe on a copy stream, two layers
ahead of the compute stream (CacheBlend explainer, "Pipelined design"; the review's Llama-70B
example, where recompute rather than loading bounds a layer).

T_blend of a step is timed with HIP events from the first fetch enqueue (copy stream) to the
end of the last layer (compute stream); steps run one at a time (each prefill alone, synchronized
before the next starts).  value = context tokens / s = N_ctx * steps / wall time of the timed
steps.  Model weights, token ids and the chunk store are resident (HBM / pinned host) before
timing starts; the cached KV crosses PCIe inside every step.

Extra fields of the same JSON line: the 4K-context Llama-70B prompt on the same engine; the
16K prompt with the cached KV already in HBM and its full recompute (graph replay); per-layer
load / recompute / overlap; the Qwen2.5-1.5B-shaped workload (pinned-host single prefill,
HBM-resident graph replay and the rows built beyond the hot path: store, decode, controller,
selection variants, int8 weights); the Mistral-7B-shaped ratio sweep; Yi-34B-shaped bf16 and
int8-weight prefills.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--only-headline] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_PCIE_GBS = 64.0       # PCIe 5.0 x16, one direction
DECODE_ROWS = 32           # fused-KV rows kept free after the prompt for the decode steps
DEVICE_SEED = 1234         # seed of the weights drawn on the device (layer l: DEVICE_SEED + l)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def schedule_text(sched):
    """'1.0, 0.30, 0.15 x 26' for a schedule whose last ratio repeats."""
    s = [float(x) for x in sched]
    n_tail = 1
    while n_tail < len(s) and s[-n_tail - 1] == s[-1]:
        n_tail += 1
    head = s[: len(s) - n_tail]
    parts = [f"{x:.2f}" if x < 1 else "1.0" for x in head]
    tail = f"{s[-1]:.2f}" if s[-1] < 1 else "1.0"
    return ", ".join(parts + [tail + (f" x {n_tail}" if n_tail > 1 else "")])


def describe(wl, where: str, weights: str):
    sh = wl.shape
    lens = sorted(set(wl.chunk_lens))
    chunks = (f"{len(wl.chunk_lens)}x{lens[0]}-token" if len(lens) == 1
              else f"{len(wl.chunk_lens)} ragged ({min(lens)}-{max(lens)} token)")
    return (f"{wl.name}: {sh.name}-shaped blended prefill, {sh.n_layers} layers, d_model {sh.d_model}, "
            f"{sh.n_q_heads}/{sh.n_kv_heads} heads of {sh.head_dim}, FFN {sh.ffn_dim}, {sh.dtype}; {chunks} cached "
            f"chunks + {wl.n_query}-token query, recompute {schedule_text(wl.schedule)}; {where}; {weights}")


def attention_flops(shape, records):
    """4 * H_q * d_h * sum over kept rows of (position + 1), per layer."""
    return [4.0 * shape.n_q_heads * shape.head_dim * float((r.new_sel.astype(np.int64) + 1).sum()) for r in records]


def sync():
    import torch
    torch.cuda.synchronize()


_STREAMS = []


def streams():
    """The one (compute, copy) stream pair every engine of this process uses.  HIP spreads
    streams over a few hardware queues (4 here) in creation order, so streams made per engine
    can land on one queue, which then runs the copy stream's fetches and the compute stream's
    kernels one after the other; one pair made first keeps them on separate queues."""
    import torch
    if not _STREAMS:
        _STREAMS.extend([torch.cuda.Stream(), torch.cuda.Stream()])
    return tuple(_STREAMS)


def device_engine(sh, max_tokens, int8=False):
    """An engine whose weights are drawn on the device (N(0, 0.02), layer l seeded DEVICE_SEED + l)."""
    from rag_kv_cache_amd.pipeline import Engine
    eng = Engine(sh, max_tokens=max_tokens, streams=streams())
    for l in range(sh.n_layers):
        eng.load_layer_device(l, DEVICE_SEED + l + 1, int8=int8)
    eng.load_embedding_device(DEVICE_SEED)
    sync()
    return eng


def graph_ms(eng, fn, steps, warmup):
    """Capture fn (a whole step enqueued on the compute stream) as a HIP graph and time its
    replays: ms per replay over `steps` replays after `warmup`."""
    import torch
    from rag_kv_cache_amd.pipeline import capture_step
    fn()
    g = capture_step(eng, fn)
    cs = eng.compute
    with torch.cuda.stream(cs):
        for _ in range(warmup):
            g.replay()
    cs.synchronize()
    sync()
    t0 = time.perf_counter()
    with torch.cuda.stream(cs):
        for _ in range(steps):
            g.replay()
    cs.synchronize()
    sync()
    ms = (time.perf_counter() - t0) / steps * 1e3
    del g
    return ms


def kernel_table(eng, prof_steps, attn_work, pcie_peak):
    """Per-kernel HIP-event durations (cb_profile) over `prof_steps` profiled steps, with each
    kernel's algorithmic rate against its roofline."""
    from rag_kv_cache_amd import _lib as L
    mfma = (L.CB_K_GEMM_KV, L.CB_K_GEMM_Q, L.CB_K_ATTN, L.CB_K_GEMM_O, L.CB_K_GEMM_GATE_UP, L.CB_K_GEMM_DOWN)
    kernels = {}
    for kid, name in enumerate(L.KERNEL_NAMES):
        ms, n, work = L.cb_profile_read(eng.ctx, kid)
        if n == 0:
            continue
        if kid == L.CB_K_ATTN:
            work = attn_work * prof_steps
        bound = "mfma" if kid in mfma else ("pcie" if kid == L.CB_K_FETCH else "hbm")
        scale = 1e12 if bound == "mfma" else 1e9
        rate = work / (ms * 1e-3) / scale if ms > 0 else 0.0
        peak = {"mfma": PEAK_BF16_TFLOPS, "hbm": PEAK_HBM_GBS, "pcie": pcie_peak}[bound]
        kernels[name] = {"ms_total_per_step": round(ms / prof_steps, 4), "launches_per_step": n // prof_steps,
                         "us_per_launch": round(ms * 1e3 / n, 2), "bound": bound, "achieved": round(rate, 2),
                         "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "peak": peak,
                         "frac": round(rate / peak, 4), "work_per_launch": work / n}
    return kernels


def mfma_busy_from_profiles(workload):
    """{kernel name: MFMA-busy share of SIMD cycles} over one step's launches of each product and
    of the attention, from the committed rocprofv3 counter summary
    profiles/mfma_busy_by_kernel_<workload>.txt, or {} if it is missing or was taken on other
    kernel sources."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"mfma_busy_by_kernel_{workload}.txt")
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    for src, digest in re.findall(r"source_sha256 (\S+): ([0-9a-f]{64})", text):
        p = os.path.join(ROOT, src)
        if not os.path.exists(p) or hashlib.sha256(open(p, "rb").read()).hexdigest() != digest:
            return {}
    return {k: float(v) for k, v in re.findall(r"^(\w+): last \d+ dispatches: .*?mfma_busy ([\d.]+)", text, re.M)}


def traffic_from_profiles(kernel, workload, launches_per_step):
    """HBM bytes per launch of `kernel` averaged over one step of `workload`, from the committed
    rocprofv3 counter summary profiles/<kernel>_<workload>_traffic.txt (FETCH_SIZE and WRITE_SIZE
    per dispatch, each scaled by what it reads for a plain device copy; the step's launches are
    the last ones of the profiled run), or None if that summary is missing, covers another
    number of launches per step, or was taken on another version of the kernel's source."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    for src, digest in re.findall(r"source_sha256 (\S+): ([0-9a-f]{64})", text):
        p = os.path.join(ROOT, src)
        if not os.path.exists(p) or hashlib.sha256(open(p, "rb").read()).hexdigest() != digest:
            return None
    m = re.search(r"step average over the last (\d+) launches: ([\d.]+) MB per launch", text)
    if not m or int(m.group(1)) != launches_per_step:
        return None
    return round(float(m.group(2)) * 1e6)


def run_prompt_pinned(eng, store, wl, steps, warmup, profile=False, overlap=False, hbm=False, full=False,
                      full_steps=2):
    """One prompt on an engine whose chunk store holds the prompt's chunks: the blended prefill
    with the cached KV fetched from the store's pinned arena, timed one prefill at a time (the
    contract's steps), plus optionally a kernel profile, per-layer load / recompute / overlap,
    the same prefill with the cached KV already in HBM (graph replay) and the full recompute
    (ratio 1 at every layer, graph replay)."""
    import torch
    import fixtures as F
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    sh = wl.shape
    chunks = F.chunk_tokens(wl)
    tokens = F.all_tokens(wl)
    offs = [int(o) for o in F.chunk_offsets(wl)]
    slots = store.lookup_prompt(chunks, hold=True)
    assert slots is not None, "the chunk store lacks a chunk of the prompt"
    hc = store.host_cache(slots)
    n_tok = wl.n_tokens
    buf = make_buffers(eng, n_tok, len(chunks))
    fused = [(eng.kv_empty(n_tok), eng.kv_empty(n_tok)) for _ in range(sh.n_layers)]
    rec = run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, host_cache=hc, record="sets")
    sync()
    attn_fl = attention_flops(sh, rec.records)
    kept = [len(r.new_sel) for r in rec.records]

    def prefill(layer_events=None):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(eng.copy)   # T_blend starts at the first fetch enqueue
        run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, host_cache=hc, upload_inputs=False,
                   layer_events=layer_events)
        e1.record(eng.compute)
        return e0, e1

    for _ in range(warmup):
        prefill()
        sync()
    sync()
    evs = []
    t0 = time.perf_counter()
    for _ in range(steps):
        evs.append(prefill())
        sync()  # each prefill alone: the next one's fetch does not overlap this one's compute
    wall = time.perf_counter() - t0
    t_blend = [a.elapsed_time(b) for a, b in evs]
    layer_ev = []
    prefill(layer_ev)
    sync()
    per_layer = [layer_ev[i].elapsed_time(layer_ev[i + 1]) for i in range(len(layer_ev) - 1)]
    out = {"n_ctx": wl.n_ctx, "n_query": wl.n_query, "steps": steps, "warmup": warmup,
           "wall_ms_per_step": round(wall / steps * 1e3, 4),
           "context_tokens_per_s": round(wl.n_ctx * steps / wall, 1),
           "t_blend_ms": {"median": round(float(np.median(t_blend)), 4), "min": round(min(t_blend), 4),
                          "max": round(max(t_blend), 4)},
           "per_layer_ms": {"layer1": round(per_layer[0], 4), "layer2": round(per_layer[1], 4),
                            "steady_median": round(float(np.median(per_layer[2:])), 4),
                            "steady_min": round(float(np.min(per_layer[2:])), 4),
                            "steady_max": round(float(np.max(per_layer[2:])), 4)},
           "kept_rows_per_layer": kept[:3] + ["..."],
           "host_kv_bytes_per_step": int(2 * sh.n_layers * wl.n_ctx * sh.n_kv_heads * sh.head_dim * 2)}
    log(f"{wl.name}: pinned-host blended prefill {out['wall_ms_per_step']:.3f} ms/step (T_blend median "
        f"{out['t_blend_ms']['median']:.3f} ms), {out['context_tokens_per_s']:,.0f} context tokens/s; layer 1 "
        f"{per_layer[0]:.3f} ms, steady {out['per_layer_ms']['steady_median']:.3f} ms")
    if profile:
        L.cb_profile_enable(eng.ctx, True)
        prefill()
        sync()
        L.cb_profile_enable(eng.ctx, False)
        out["kernels"] = kernel_table(eng, 1, sum(attn_fl), PEAK_PCIE_GBS)
        for name in ("fetch", "rope_delta"):  # the fetch and its position update run on the copy stream
            if name in out["kernels"]:
                out["kernels"][name]["stream"] = ("copy: beside the compute stream's kernels, so its event time "
                                                  "includes waiting for CUs they hold")
        out["attention_flops_per_step"] = sum(attn_fl)
    if overlap:
        out["per_layer_overlap"] = run_overlap(eng, buf, tokens, offs, wl, fused, hc, reps=2)
    if hbm:
        cache, _ = build_chunk_caches(eng, chunks)
        ms = graph_ms(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache,
                                              upload_inputs=False), steps, warmup)
        out["hbm_resident"] = {"ms_per_step": round(ms, 4), "context_tokens_per_s": round(wl.n_ctx / ms * 1e3, 1),
                               "note": "cached KV already in HBM (position update of every layer in one launch), "
                                       "graph replay"}
        log(f"{wl.name}: cached KV in HBM, graph replay {ms:.3f} ms/step")
        del cache
    if full:
        full_sched = [1.0] * sh.n_layers
        ms = graph_ms(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, full_sched, fused,
                                              upload_inputs=False), full_steps, 1)
        out["full_recompute"] = {"ms_per_step": round(ms, 4), "speedup_of_blend": round(ms / out["wall_ms_per_step"], 3),
                                 "note": "ratio 1 at every layer (every row recomputed, no cache), graph replay"}
        log(f"{wl.name}: full recompute {ms:.3f} ms/step ({ms / out['wall_ms_per_step']:.2f}x the blended prefill)")
    for sl in slots:
        store.release(sl)
    del buf, fused
    torch.cuda.empty_cache()
    return out


def run_headline(args):
    """The Llama-70B-shaped workload: 16K prompt (value) and 4K prompt on one engine."""
    import fixtures as F
    from rag_kv_cache_amd.pipeline import ChunkStore, produce_chunks
    import torch
    wl = F.get_config(args.config)
    sh = wl.shape
    # the 4K prompt of the same shape: its chunks are the first chunks of the 16K prompt
    small = {"l70_16k": "l70_4k"}.get(args.config)
    t0 = time.perf_counter()
    eng = device_engine(sh, wl.n_tokens + DECODE_ROWS)
    log(f"{wl.name}: {sh.n_layers} layers of weights drawn on the device in {time.perf_counter() - t0:.1f} s")
    from rag_kv_cache_amd import _lib as L
    L.cb_set_fetch_mode(eng.ctx, {"auto": L.CB_FETCH_AUTO, "kernel": L.CB_FETCH_KERNEL,
                                  "copy": L.CB_FETCH_COPY}[args.fetch])
    chunks = F.chunk_tokens(wl)
    store = ChunkStore(eng, max(wl.chunk_lens), len(chunks) + 2, pinned=True)
    t0 = time.perf_counter()
    produce_chunks(eng, store, chunks)
    t_prod = time.perf_counter() - t0
    log(f"{wl.name}: chunk producer filled the pinned store in {t_prod:.1f} s")
    res = run_prompt_pinned(eng, store, wl, args.steps, args.warmup, profile=True,
                            overlap=not args.only_headline, hbm=not args.only_headline,
                            full=not args.only_headline, full_steps=max(2, args.steps // 8))
    res["producer_context_tokens_per_s"] = round(wl.n_ctx / t_prod, 1)
    other = None
    if small and not args.only_headline:
        wl4 = F.get_config(small)
        other = run_prompt_pinned(eng, store, wl4, args.steps, args.warmup, profile=True, full=True,
                                  full_steps=max(2, args.steps // 4))
        other["workload"] = describe(wl4, "cached KV in pinned host memory (chunk store), fetched two layers ahead",
                                     "weights drawn on the device")
    store.close()
    eng.close()
    del eng
    torch.cuda.empty_cache()
    return wl, res, other


def run_controller(eng, buf, tokens, offs, wl, fused, host, full_ms, overlap, steps):
    """The loading controller on this GPU, two ways, each followed by the pinned-host prefill run
    at the ratio it plans (layer 1 stays at 1):
      * cb_plan_ratio (the explainer's model): the load bandwidth of a whole step's cached KV
        fetched alone, and the full prefill split evenly over the layers and tokens;
      * cb_plan_ratio_measured: a layer's load time from the per-layer fetch measurement, a
        layer's recompute time measured at ratio 1 (every row) and at ratio 0 (no context row:
        the fixed part), the first layer at its time in the pipelined run, the first filtering
        layer's extra cost (scoring every context row) measured at ratio 0, and the contention
        of a fetch running beside the compute: the excess of each layer (after the first two)
        over max(T_load, T_recompute), summed, over the summed min(T_load, T_recompute).  The
        contention depends on the operating point (a compute-bound pipeline lets the copy
        stream run ahead and finish early, a balanced one keeps the fetch beside every layer),
        so it is taken first from the workload's pipelined run, then from pipelined runs at the
        planned ratio (calibration runs, not timed ones): the plan is made again with the
        contention and the recompute time measured there, and calibrated again at its new ratio
        until it lands on a ratio already calibrated; the plan's predicted time is the model's
        at that ratio with that ratio's own calibration.
    Both with a ratio floor of 5% (below the workload's 15%, so that the plan is not just the
    floor) and no ceiling; each plan's prefill is timed alone, like the headline (events from the
    first fetch enqueue to the last layer's end, median of the runs)."""
    import torch
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import run_layers
    sh = wl.shape
    nl = sh.n_layers
    kv_layer_tok = 2 * sh.n_kv_heads * sh.head_dim * 2
    kv_layer = wl.n_ctx * kv_layer_tok
    r_min, r_max = 0.05, 1.0

    def layer_times(sched, reps=3):
        rows = []
        for r in range(reps + 1):
            evs = []
            run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, upload_inputs=False, cache=None,
                       layer_events=evs)
            eng.compute.synchronize()
            if r:
                rows.append([evs[i].elapsed_time(evs[i + 1]) for i in range(nl)])
        return np.median(np.array(rows), axis=0) * 1e-3

    def run_plan(plan):
        sched = [1.0] + [float(plan.ratio) if plan.load else 1.0] * (nl - 1)
        kw = dict(host_cache=host) if plan.load else dict(cache=None)
        n = max(3, steps // 2)
        ms = []
        for r in range(n + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(eng.copy)
            run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, upload_inputs=False, **kw)
            e1.record(eng.compute)
            torch.cuda.synchronize()
            if r >= 2:
                ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    def summary(plan, ms):
        return {"load": bool(plan.load), "ratio": round(float(plan.ratio), 4),
                "t_load_layer_ms": round(plan.t_load_layer * 1e3, 4),
                "t_recompute_layer_ms": round(plan.t_recompute_layer * 1e3, 4),
                "break_even_GBps": round(plan.break_even_bandwidth / 1e9, 2),
                "predicted_ms_per_step": round(plan.t_total * 1e3, 4), "measured_ms_per_step": round(ms, 4),
                "context_tokens_per_s": round(wl.n_ctx / ms * 1e3, 1)}

    # the explainer's model
    load_s = sum(overlap["t_load_ms"]) * 1e-3
    bw = nl * kv_layer / load_s
    pre = full_ms * 1e-3 / wl.n_tokens
    even = L.cb_plan_ratio(wl.n_ctx, nl, kv_layer_tok, bw, pre, 0.0, r_min, r_max)
    even_ms = run_plan(even)
    # the measured model (the fused buffers hold every layer's re-rotated cache after a fetch pass)
    t_full = layer_times([1.0] * nl)
    t_zero = layer_times([1.0] + [0.0] * (nl - 1))
    t_full_l = float(np.median(t_full[1:]))
    t_fixed_l = min(float(np.median(t_zero[2:])), t_full_l)
    t_select = max(0.0, float(t_zero[1]) - t_fixed_l)
    t_load_l = float(np.median(overlap["t_load_ms"])) * 1e-3
    def contention_of(t_ov, t_rec):
        tl_ = np.array(overlap["t_load_ms"][2:]) * 1e-3
        tr_, to_ = np.asarray(t_rec[2:]), np.asarray(t_ov[2:])
        return float(np.maximum(to_ - np.maximum(tl_, tr_), 0.0).sum() / np.minimum(tl_, tr_).sum())

    contention0 = contention_of(np.array(overlap["t_overlapped_ms"]) * 1e-3, np.array(overlap["t_recompute_ms"]) * 1e-3)
    t_first = float(overlap["t_overlapped_ms"][0]) * 1e-3  # the pipelined first layer (waits for fetches)

    def plan(k, t_fix):
        return L.cb_plan_ratio_measured(nl, kv_layer, kv_layer / t_load_l, 0.0, t_first, t_full_l, t_fix, r_min,
                                        r_max, t_select_layer=t_select, contention=k)

    def calibrate(r0):
        """Per-layer times at ratio r0, pipelined and alone: the contention there, and the
        recompute line redrawn through (r0, T_recompute alone) and (1, t_full) (small ratios cost
        more than the line from ratio 0: tile rounding of the few kept rows)."""
        sched = [1.0] + [r0] * (nl - 1)
        t_alone = layer_times(sched)
        rows = []
        for r in range(3):
            evs = []
            run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, upload_inputs=False, host_cache=host,
                       layer_events=evs)
            eng.compute.synchronize()
            rows.append([evs[i].elapsed_time(evs[i + 1]) for i in range(nl)])
        t_pipe = np.median(np.array(rows), axis=0) * 1e-3
        k = contention_of(t_pipe, t_alone)
        t_r0 = float(np.median(t_alone[2:]))
        t_fix = t_fixed_l
        if r0 < 1.0 and t_r0 < t_full_l:
            t_fix = max(0.0, t_r0 - r0 * (t_full_l - t_r0) / (1.0 - r0))
        return k, t_fix, {"ratio": round(r0, 4), "t_recompute_alone_median_ms": round(t_r0 * 1e3, 4),
                          "t_layer_pipelined_median_ms": round(float(np.median(t_pipe[2:])) * 1e3, 4),
                          "sum_pipelined_ms": round(float(t_pipe.sum()) * 1e3, 4),
                          "t_fixed_layer_redrawn_ms": round(t_fix * 1e3, 4)}

    # calibration at the planned ratio, then the plan is made again with what was measured there,
    # until the plan lands on a ratio already calibrated (at most four calibrations; the small
    # ratios' cost steps can make two ratios point at each other).  The plan's time is then the
    # model's at that ratio with that ratio's own calibration.
    meas = plan(contention0, t_fixed_l)
    contention, calibs, cal_at = contention0, [], {}
    key = lambda r: int(round(r * wl.n_ctx))  # kept context rows
    while meas.load and len(calibs) < 4:
        r0 = float(meas.ratio)
        if key(r0) in cal_at:
            break
        contention, t_fixed_c, cal = calibrate(r0)
        calibs.append(cal)
        cal_at[key(r0)] = (contention, t_fixed_c, cal)
        meas = plan(contention, t_fixed_c)
    calib = None
    if meas.load and key(float(meas.ratio)) in cal_at:
        r_star = float(meas.ratio)
        contention, t_fixed_c, calib = cal_at[key(r_star)]
        meas = L.cb_plan_ratio_measured(nl, kv_layer, kv_layer / t_load_l, 0.0, t_first, t_full_l, t_fixed_c, r_star,
                                        r_star, t_select_layer=t_select, contention=contention)
    elif calibs:
        calib = calibs[-1]
    meas_ms = run_plan(meas)
    log(f"controller (even split): load {bw / 1e9:.1f} GB/s, ratio {even.ratio:.3f}, predicted "
        f"{even.t_total * 1e3:.3f} ms, measured {even_ms:.3f} ms/step")
    log(f"controller (measured layer times: first {t_first * 1e3:.3f}, first filter +{t_select * 1e3:.3f}, full "
        f"{t_full_l * 1e3:.3f}, fixed {t_fixed_l * 1e3:.3f}, load {t_load_l * 1e3:.3f} ms, contention "
        f"{contention0:.3f} at the workload's ratio, {contention:.3f} at the plan's): ratio {meas.ratio:.3f} "
        f"(load={meas.load}), predicted {meas.t_total * 1e3:.3f} ms, measured {meas_ms:.3f} ms/step")
    return {"r_min": r_min, "r_max": r_max,
            "even_split": dict(summary(even, even_ms), load_bandwidth_GBps=round(bw / 1e9, 2),
                               prefill_us_per_token=round(pre * 1e6, 4)),
            "measured_layers": dict(summary(meas, meas_ms), t_first_ms=round(t_first * 1e3, 4),
                                    t_select_ms=round(t_select * 1e3, 4), t_full_layer_ms=round(t_full_l * 1e3, 4),
                                    t_fixed_layer_ms=round(t_fixed_l * 1e3, 4),
                                    contention_workload_ratio=round(contention0, 4), contention=round(contention, 4),
                                    calibration_at_plan=calib, calibrations=calibs,
                                    prediction_error=round(meas.t_total * 1e3 / meas_ms - 1, 4)),
            "schedule": "1.0, then the planned ratio (pinned-host cache fetched two layers ahead; eager launches; "
                        "each prefill timed alone)"}


def _fetch_layer(eng, buf, host, offs, l, fused):
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import _ptr
    n_chunks = len(offs) - 1
    L.cb_fetch_layer(eng.ctx, l, [_ptr(host[l][c][0]) for c in range(n_chunks)],
                     [_ptr(host[l][c][1]) for c in range(n_chunks)], offs, n_chunks,
                     _ptr(buf.offsets), _ptr(fused[l][0]), _ptr(fused[l][1]))


def run_overlap(eng, buf, tokens, offs, wl, fused, host, reps: int = 5, eps_ms: float = 0.02, eps_rel: float = 0.01):
    """Per-layer T_load, T_recompute and T_overlapped of the pinned-host prefetched prefill, medians
    over `reps` runs:
      * T_load[l]: layer l's fetch alone (cached K/V of every chunk over PCIe + position update),
        HIP events around each launch on the copy stream, every layer fetched back to back with
        no compute running;
      * T_recompute[l]: layer l's compute alone (blend + rest), events on the compute stream, the
        fused buffers already holding the re-rotated cache (no fetch);
      * T_overlapped[l]: layer l on the compute stream in the pipelined run (fetches two layers
        ahead on the copy stream), including any wait for its fetch.
    The pipeline claim is checked per layer as T_overlapped <= max(T_load, T_recompute) + eps, with
    eps = eps_ms, and again with eps = max(eps_ms, eps_rel * max(...)) for layers of several ms."""
    import torch
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import run_layers
    nl = wl.shape.n_layers
    xs, cs = eng.copy, eng.compute
    loads, recs, ovs = [], [], []

    def layer_times(kw):
        evs = []
        run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, upload_inputs=False,
                   layer_events=evs, **kw)
        cs.synchronize()
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(nl)]

    for r in range(reps + 1):  # the first round warms up
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)]
        ev[0].record(xs)
        for l in range(nl):
            _fetch_layer(eng, buf, host, offs, l, fused)
            ev[l + 1].record(xs)
        for l in range(nl):
            L.cb_synchronize(eng.ctx, l)
        xs.synchronize()
        cs.synchronize()
        lt = [ev[i].elapsed_time(ev[i + 1]) for i in range(nl)]
        # the fused buffers now hold every layer's re-rotated cache: compute alone over them
        rt = layer_times(dict(cache=None))
        ot = layer_times(dict(host_cache=host))
        if r:
            loads.append(lt)
            recs.append(rt)
            ovs.append(ot)
    med = lambda rows: [float(np.median(c)) for c in zip(*rows)]
    t_load, t_rec, t_ov = med(loads), med(recs), med(ovs)
    excess = [t_ov[l] - max(t_load[l], t_rec[l]) for l in range(nl)]
    steady = list(range(3, nl)) if nl > 4 else list(range(nl))
    ok = [l for l in range(nl) if excess[l] <= eps_ms]
    ok_rel = [l for l in range(nl) if excess[l] <= max(eps_ms, eps_rel * max(t_load[l], t_rec[l]))]
    log(f"overlap (steady medians): load {np.median([t_load[l] for l in steady]):.4f}, recompute "
        f"{np.median([t_rec[l] for l in steady]):.4f}, overlapped {np.median([t_ov[l] for l in steady]):.4f} ms; "
        f"{len(ok)}/{nl} layers within max(load, recompute) + {eps_ms} ms, {len(ok_rel)}/{nl} within "
        f"+ max({eps_ms} ms, {eps_rel:.0%}); sum overlapped {sum(t_ov):.3f} vs sum max "
        f"{sum(max(a, b) for a, b in zip(t_load, t_rec)):.3f} ms")
    r4 = lambda v: [round(x, 4) for x in v]
    return {"t_load_ms": r4(t_load), "t_recompute_ms": r4(t_rec), "t_overlapped_ms": r4(t_ov),
            "steady_median_ms": {"load": round(float(np.median([t_load[l] for l in steady])), 4),
                                 "recompute": round(float(np.median([t_rec[l] for l in steady])), 4),
                                 "overlapped": round(float(np.median([t_ov[l] for l in steady])), 4)},
            "sum_ms": {"load": round(sum(t_load), 4), "recompute": round(sum(t_rec), 4),
                       "overlapped": round(sum(t_ov), 4),
                       "max_per_layer": round(sum(max(a, b) for a, b in zip(t_load, t_rec)), 4)},
            "check": {"eps_ms": eps_ms, "layers_within": len(ok), "layers": nl,
                      "eps_rel": eps_rel, "layers_within_rel": len(ok_rel),
                      "sum_overlapped_over_sum_max": round(sum(t_ov) / sum(max(a, b) for a, b in zip(t_load, t_rec)), 4),
                      "max_excess_ms": round(max(excess), 4),
                      "steady_median_excess_ms": round(float(np.median([excess[l] for l in steady])), 4)},
            "note": "per-layer medians over %d runs; T_load: each layer's fetch alone on the copy stream; "
                    "T_recompute: compute alone on fused buffers that already hold the cache" % reps}


def run_reuse(eng, buf, tokens, offs, wl, fused, cache, steps):
    """Lower bounds on the same GPU and kernels (HBM-resident cache, graph replay as for value):
    full KV reuse as ratio 0 from layer 2 (layer 1 recomputes every row, later layers only the
    query rows), and no context row recomputed at any layer (only the query rows run through
    the model over the re-rotated caches)."""
    import torch
    from rag_kv_cache_amd.pipeline import capture_step, run_layers
    sh = wl.shape
    cs = eng.compute
    q_only = list(range(wl.n_ctx, wl.n_tokens))

    def timed(sched, init=None):
        run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, cache=cache, upload_inputs=init is None,
                   initial_sel=init)
        g = capture_step(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, cache=cache,
                                                 upload_inputs=False, initial_sel=init, sel_uploaded=True))
        with torch.cuda.stream(cs):
            for _ in range(3):
                g.replay()
        cs.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(cs):
            for _ in range(steps):
                g.replay()
        cs.synchronize()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    reuse_ms = timed([1.0] + [0.0] * (sh.n_layers - 1))
    query_ms = timed([1.0] * sh.n_layers, q_only)
    buf.tokens[: wl.n_tokens].copy_(torch.from_numpy(np.asarray(tokens, np.int32)))
    buf.offsets[: len(offs)].copy_(torch.tensor(offs, dtype=torch.int32))
    torch.cuda.synchronize()
    log(f"full KV reuse (ratio 0 from layer 2): {reuse_ms:.3f} ms/step; query rows only: {query_ms:.3f} ms/step")
    return {"ratio0_from_layer2_ms": round(reuse_ms, 4), "query_rows_only_ms": round(query_ms, 4),
            "note": "graph replay; HBM-resident chunk caches; the position update of every cached row is included"}


def run_peaks(eng):
    """This GPU's own ceilings next to the published ones: a device-to-device copy (torch's copy
    kernel, read + write bytes), a pinned host-to-device copy (copy engine), and a large bf16
    product through the vendor BLAS (torch.mm, 8192^3)."""
    import torch
    dv = eng.device
    st = torch.cuda.current_stream(dv)

    def timed(fn, reps):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    nb = 1 << 30
    src = torch.empty(nb // 2, dtype=torch.bfloat16, device=dv)
    dst = torch.empty_like(src)
    copy_gbs = 2 * nb / timed(lambda: dst.copy_(src), 20) / 1e9
    del src, dst
    hb = 256 << 20
    h = torch.empty(hb, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(hb, dtype=torch.uint8, device=dv)
    h2d_gbs = hb / timed(lambda: d.copy_(h, non_blocking=True), 10) / 1e9
    del h, d
    m = 8192
    a = torch.randn(m, m, device=dv, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dv, dtype=torch.bfloat16)
    c = torch.empty(m, m, device=dv, dtype=torch.bfloat16)
    mm_tf = 2 * m ** 3 / timed(lambda: torch.mm(a, b, out=c), 20) / 1e12
    del a, b, c
    torch.cuda.synchronize()
    log(f"peaks on this GPU: device copy {copy_gbs:.0f} GB/s, pinned H2D {h2d_gbs:.1f} GB/s, "
        f"bf16 mm {mm_tf:.0f} TFLOP/s")
    return {"device_copy_GBps": round(copy_gbs, 1), "pinned_h2d_GBps": round(h2d_gbs, 2),
            "bf16_mm_8192_TFLOPs": round(mm_tf, 1),
            "published": {"hbm_GBps": PEAK_HBM_GBS, "bf16_dense_TFLOPs": PEAK_BF16_TFLOPS, "pcie5_x16_GBps": 64.0},
            "note": "torch copy_ (read + write bytes over 1 GiB), torch copy_ from 256 MiB pinned host memory, "
                    "torch.mm bf16 8192 x 8192 x 8192"}


def run_int8(wl, steps, warmup):
    """The same blended prefill with int8 weights (per-output-channel scales; the same float32
    draws quantized), HBM-resident caches, graph replay: ms per step and the gate/up product's
    share."""
    import torch
    import fixtures as F
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, capture_step, make_buffers, run_layers
    sh = wl.shape
    eng = Engine(sh, max_tokens=wl.n_tokens + 8, streams=streams())
    for l in range(sh.n_layers):
        eng.load_layer_int8(l, F.layer_weights_int8(sh, l + 1))
    eng.load_embedding(F.embedding(sh))
    chunks = F.chunk_tokens(wl)
    tokens = F.all_tokens(wl)
    offs = [int(o) for o in F.chunk_offsets(wl)]
    cache, _ = build_chunk_caches(eng, chunks)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = [(eng.kv_empty(wl.n_tokens), eng.kv_empty(wl.n_tokens)) for _ in range(sh.n_layers)]
    run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache)
    g = capture_step(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache,
                                             upload_inputs=False))
    cs = eng.compute
    with torch.cuda.stream(cs):
        for _ in range(warmup):
            g.replay()
    cs.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(cs):
        for _ in range(steps):
            g.replay()
    cs.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    L.cb_profile_enable(eng.ctx, True)
    run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache, upload_inputs=False)
    cs.synchronize()
    L.cb_profile_enable(eng.ctx, False)
    gu_ms, gu_n, _ = L.cb_profile_read(eng.ctx, L.CB_K_GEMM_GATE_UP)
    del g
    eng.close()
    log(f"int8 weights: {ms:.3f} ms/step, gate/up {gu_ms * 1e3 / max(gu_n, 1):.1f} us per launch")
    return {"ms_per_step": round(ms, 4), "context_tokens_per_s": round(wl.n_ctx / ms * 1e3, 1),
            "gate_up_us_per_launch": round(gu_ms * 1e3 / max(gu_n, 1), 2),
            "note": "int8 weights, one float32 scale per output channel, bf16 activations; graph replay"}


def run_variants(eng, buf, tokens, offs, wl, fused, cache, steps):
    """The selection variants of the KVBoost page on the same workload (HBM-resident cache,
    eager launches): the cosine deviation score with the same schedule, and the spatial seam
    set (16 positions before every chunk boundary + the query) kept at every layer."""
    import torch
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import run_layers
    sh = wl.shape
    n = max(3, steps // 2)

    def timed(**kw):
        for _ in range(2):
            run_layers(eng, buf, tokens, offs, wl.n_query, kw.get("sched", wl.schedule), fused, cache=cache,
                       upload_inputs=False, initial_sel=kw.get("initial_sel"))
        eng.compute.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            run_layers(eng, buf, tokens, offs, wl.n_query, kw.get("sched", wl.schedule), fused, cache=cache,
                       upload_inputs=False, initial_sel=kw.get("initial_sel"))
        eng.compute.synchronize()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e3

    L.cb_set_score_mode(eng.ctx, L.CB_SCORE_COSINE)
    cos_ms = timed()
    L.cb_set_score_mode(eng.ctx, L.CB_SCORE_L2)
    seam = L.cb_seam_select(offs, len(offs) - 1, wl.n_query, 16)
    seam_ms = timed(sched=[1.0] * sh.n_layers, initial_sel=seam)
    # leave the token ids on the device as the default runs expect them
    buf.tokens[: wl.n_tokens].copy_(torch.from_numpy(np.asarray(tokens, np.int32)))
    torch.cuda.synchronize()
    log(f"variants: cosine score {cos_ms:.3f} ms/step; seam set ({len(seam)} rows) {seam_ms:.3f} ms/step")
    return {"cosine_score": {"ms_per_step": round(cos_ms, 4), "context_tokens_per_s": round(wl.n_ctx / cos_ms * 1e3, 1),
                             "schedule": "1.0, 0.30, 0.15 x 26 (eager)"},
            "seam_set": {"rows": len(seam), "window": 16, "ms_per_step": round(seam_ms, 4),
                         "context_tokens_per_s": round(wl.n_ctx / seam_ms * 1e3, 1),
                         "schedule": "the seam set at every layer (eager)"}}


def run_decode(eng, buf, tokens, offs, wl, fused, cache):
    """Generation with the fused KV after one blended prefill: single-token decode steps through
    all layers (given token ids; no LM head), ms per token, eager launches."""
    import torch
    from rag_kv_cache_amd.pipeline import decode, run_layers
    run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache, upload_inputs=False)
    eng.compute.synchronize()
    n = wl.n_tokens
    steps = 16
    assert steps + 2 <= DECODE_ROWS
    for i in range(2):  # warmup (appends rows n, n+1; overwritten below)
        decode(eng, buf, [i + 1], n + i, fused)
    eng.compute.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        decode(eng, buf, [(7 * i) % wl.shape.vocab], n + i, fused)
    eng.compute.synchronize()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    buf.tokens[: wl.n_tokens].copy_(torch.from_numpy(np.asarray(tokens, np.int32)))
    torch.cuda.synchronize()
    log(f"decode: {ms:.3f} ms/token ({steps} single-token steps after the blended prefill)")
    return {"ms_per_token": round(ms, 4), "tokens_per_s": round(1e3 / ms, 1), "steps": steps,
            "context_rows": n, "note": "single-token steps on the fused KV, eager launches, given token ids"}


def run_store(eng, buf, tokens, offs, wl, fused, steps):
    """Chunk-cache producer into a pinned host store, prompt lookup, and the blended prefill
    fetched from the store's arena (same fetch path as the separately pinned caches)."""
    import torch
    from rag_kv_cache_amd.pipeline import ChunkStore, produce_chunks, run_layers
    import fixtures as F
    sh = wl.shape
    chunks = F.chunk_tokens(wl)
    store = ChunkStore(eng, max(wl.chunk_lens), len(chunks) + 2, pinned=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    produce_chunks(eng, store, chunks)
    t_prod = time.perf_counter() - t0
    reps = 200
    t0 = time.perf_counter()
    for _ in range(reps):
        slots = store.lookup_prompt(chunks, hold=True)
        for sl in slots:
            store.release(sl)
    t_look = (time.perf_counter() - t0) / (reps * len(chunks))
    slots = store.lookup_prompt(chunks, hold=True)
    hc = store.host_cache(slots)
    cs = eng.compute

    def step():
        run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, host_cache=hc, upload_inputs=False)

    for _ in range(2):
        step()
    cs.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    cs.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    st = store.stats()
    for sl in slots:
        store.release(sl)
    store.close()
    out = {"producer_context_tokens_per_s": round(wl.n_ctx / t_prod, 1),
           "producer_s": round(t_prod, 4),
           "lookup_us_per_chunk": round(t_look * 1e6, 2),
           "chunk_tokens": max(wl.chunk_lens),
           "prefill_from_store_ms": round(ms, 4),
           "store_bytes_per_chunk": int(st.slot_bytes), "index_bytes": int(st.index_bytes),
           "entries": int(st.entries)}
    log(f"chunk store: producer {out['producer_context_tokens_per_s']:.0f} tok/s, lookup "
        f"{out['lookup_us_per_chunk']:.1f} us/chunk, prefill from store {ms:.3f} ms/step")
    return out




def run_qwen(args):
    """The Qwen2.5-1.5B-shaped workload (fixture weights): pinned-host single prefill, HBM-resident
    graph replay with its per-kernel table, full recompute and lower bounds by graph replay,
    per-layer overlap, and the rows beyond the hot path (controller, selection variants, decode,
    chunk store, int8 weights)."""
    import torch
    import fixtures as F
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import ChunkStore, Engine, build_chunk_caches, make_buffers, produce_chunks, run_layers
    wl = F.get_config("qwen")
    sh = wl.shape
    chunks = F.chunk_tokens(wl)
    tokens = F.all_tokens(wl)
    offs = [int(o) for o in F.chunk_offsets(wl)]
    n_ctx, n_tok = wl.n_ctx, wl.n_tokens
    eng = Engine(sh, max_tokens=n_tok + 64, streams=streams())
    for l in range(sh.n_layers):
        eng.load_layer(l, F.layer_weights(sh, l + 1))
    eng.load_embedding(F.embedding(sh))
    cache, _ = build_chunk_caches(eng, chunks)
    # the pinned-host cache is the chunk store's arena, filled by the chunk producer (consecutive
    # slots, so each layer's chunks are adjacent and fetched in one copy per tensor)
    hstore = ChunkStore(eng, max(wl.chunk_lens), len(chunks) + 2, pinned=True)
    produce_chunks(eng, hstore, chunks)
    hslots = hstore.lookup_prompt(chunks, hold=True)
    host = hstore.host_cache(hslots)
    buf = make_buffers(eng, n_tok + DECODE_ROWS, len(chunks))
    fused = [(eng.kv_empty(n_tok + DECODE_ROWS), eng.kv_empty(n_tok + DECODE_ROWS)) for _ in range(sh.n_layers)]
    cs = eng.compute
    rec = run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache, record="sets")
    attn_fl = attention_flops(sh, rec.records)
    out = {"workload": describe(wl, "see the fields for where the cached KV lives", "fixture weights")}

    def step(**kw):
        return run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, upload_inputs=False, **kw)

    # pinned host: one prefill at a time, events from the first fetch enqueue to the last layer
    for _ in range(2):
        step(host_cache=host)
    sync()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(eng.copy)
        step(host_cache=host)
        e1.record(cs)
        sync()
        evs.append((e0, e1))
    wall = time.perf_counter() - t0
    tb = [a.elapsed_time(b) for a, b in evs]
    out["pinned_host"] = {"wall_ms_per_step": round(wall / args.steps * 1e3, 4),
                          "context_tokens_per_s": round(n_ctx * args.steps / wall, 1),
                          "t_blend_ms_median": round(float(np.median(tb)), 4),
                          "note": "cached KV in pinned host memory, fetched two layers ahead; one prefill at a time"}
    # back to back: each prefill's fetches overlap the previous prefill's compute
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(host_cache=host)
    sync()
    bb = (time.perf_counter() - t0) / args.steps * 1e3
    out["pinned_host_back_to_back_ms"] = round(bb, 4)
    log(f"qwen: pinned host {out['pinned_host']['wall_ms_per_step']:.3f} ms/prefill alone "
        f"(T_blend {out['pinned_host']['t_blend_ms_median']:.3f}), {bb:.3f} ms back to back")
    # cached KV in HBM: graph replay, and its per-kernel table
    hbm_ms = graph_ms(eng, lambda: step(cache=cache), args.steps, args.warmup)
    L.cb_profile_enable(eng.ctx, True)
    for _ in range(3):
        step(cache=cache)
    cs.synchronize()
    L.cb_profile_enable(eng.ctx, False)
    kernels = kernel_table(eng, 3, sum(attn_fl), PEAK_PCIE_GBS)
    evl = []
    step(cache=cache, layer_events=evl)
    cs.synchronize()
    per_layer = [evl[i].elapsed_time(evl[i + 1]) for i in range(len(evl) - 1)]
    out["hbm_resident"] = {"ms_per_step": round(hbm_ms, 4), "context_tokens_per_s": round(n_ctx / hbm_ms * 1e3, 1),
                           "per_layer_ms": {"layer1": round(per_layer[0], 4), "layer2": round(per_layer[1], 4),
                                            "layer3": round(per_layer[2], 4),
                                            "steady_median": round(float(np.median(per_layer[3:])), 4)},
                           "kernels": kernels, "note": "cached KV resident in HBM, graph replay"}
    log(f"qwen: HBM-resident graph replay {hbm_ms:.3f} ms/step")
    full_ms = graph_ms(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, [1.0] * sh.n_layers, fused,
                                               cache=cache, upload_inputs=False), max(3, args.steps // 2), 1)
    out["full_recompute_ms"] = round(full_ms, 4)
    out["speedup_vs_full_recompute"] = {"hbm_resident": round(full_ms / hbm_ms, 3),
                                        "pinned_host": round(full_ms / out["pinned_host"]["wall_ms_per_step"], 3),
                                        "note": "full recompute by graph replay on the same kernels"}
    log(f"qwen: full recompute {full_ms:.3f} ms/step")
    out["prefetch_per_layer"] = run_overlap(eng, buf, tokens, offs, wl, fused, host)
    out["full_reuse"] = run_reuse(eng, buf, tokens, offs, wl, fused, cache, args.steps)
    out["loading_controller"] = run_controller(eng, buf, tokens, offs, wl, fused, host, full_ms,
                                               out["prefetch_per_layer"], args.steps)
    out["selection_variants"] = run_variants(eng, buf, tokens, offs, wl, fused, cache, args.steps)
    out["decode"] = run_decode(eng, buf, tokens, offs, wl, fused, cache)
    out["chunk_store"] = run_store(eng, buf, tokens, offs, wl, fused, args.steps)
    out["peaks_measured"] = run_peaks(eng)
    for sl in hslots:
        hstore.release(sl)
    hstore.close()
    eng.close()
    del eng, cache, host, buf, fused
    torch.cuda.empty_cache()
    out["int8_weights"] = run_int8(wl, args.steps, args.warmup)
    return out


def run_hbm_shape(name, ratios, args, int8=False):
    """A shape whose cached KV stays in HBM (Mistral-7B, Yi-34B): weights drawn on the device,
    chunk caches built by the chunk producer, the blended prefill by graph replay at each ratio
    (schedule 1.0, r, r, ...) and the full recompute."""
    import torch
    import fixtures as F
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    wl = F.get_config(name)
    sh = wl.shape
    chunks = F.chunk_tokens(wl)
    tokens = F.all_tokens(wl)
    offs = [int(o) for o in F.chunk_offsets(wl)]
    eng = device_engine(sh, wl.n_tokens + 8, int8=int8)
    cache, _ = build_chunk_caches(eng, chunks)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = [(eng.kv_empty(wl.n_tokens), eng.kv_empty(wl.n_tokens)) for _ in range(sh.n_layers)]
    run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache)
    out = {"workload": describe(wl, "cached KV resident in HBM, graph replay",
                                "int8 weights (per-output-channel scales) drawn and quantized on the device"
                                if int8 else "weights drawn on the device")}
    for r in ratios:
        sched = [1.0] + [r] * (sh.n_layers - 1)
        ms = graph_ms(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, cache=cache,
                                              upload_inputs=False), args.steps, args.warmup)
        out[f"r{r:.2f}"] = {"ms_per_step": round(ms, 4), "context_tokens_per_s": round(wl.n_ctx / ms * 1e3, 1)}
        log(f"{name}{' int8' if int8 else ''}: ratio {r:.2f}: {ms:.3f} ms/step, {wl.n_ctx / ms * 1e3:,.0f} context tokens/s")
    if not int8:
        full = graph_ms(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, [1.0] * sh.n_layers, fused,
                                                upload_inputs=False), max(2, args.steps // 4), 1)
        out["full_recompute_ms"] = round(full, 4)
        log(f"{name}: full recompute {full:.3f} ms/step")
    eng.close()
    del eng, cache, buf, fused
    torch.cuda.empty_cache()
    return out


def _host_info():
    """CPU model, logical CPUs and the BLAS numpy was built with."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version', '')}".strip()
    except Exception:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas": blas}


def _oracle_layer_flops(sh, n_sel, n_keep, n_keys):
    """Flops of one oracle layer as the oracle computes them: the K/V products of the selected
    rows, Q, o-projection and FFN of the kept rows, and attention scores and sums over keys
    0 .. n_keys - 1 for every kept row (the oracle masks inside a full score matrix)."""
    d, qd, kvd, f = sh.d_model, sh.n_q_heads * sh.head_dim, sh.n_kv_heads * sh.head_dim, sh.ffn_dim
    return (2.0 * n_sel * d * 2 * kvd + 2.0 * n_keep * d * qd + 4.0 * n_keep * n_keys * qd
            + 2.0 * n_keep * qd * d + 6.0 * n_keep * d * f)


def cpu_baseline(wl, budget_s: float = 20.0):
    """The oracle (fp64 NumPy, bf16 rounding points emulated) on a bounded sample of the same
    workload: one steady layer (the kept rows at the workload's ratio, attending over the whole
    prompt) run on a fraction of its kept rows, the fraction grown until the time budget is
    used; the steady layer's time is the sample's scaled by the row fraction (every part of the
    layer is linear in the kept rows at a fixed prompt), layers 1 and 2 by the oracle's own flop
    counts relative to the steady layer.  Weights are the fixtures' layer-3 draws; the residual
    rows and the chunk caches are random values of the real shape (the oracle's cost does not
    depend on them)."""
    import fixtures as F
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    sh = wl.shape
    prec = O.Precision("bf16")
    rng = np.random.default_rng(0)
    n_ctx, n_q, n_tok = wl.n_ctx, wl.n_query, wl.n_tokens
    offs = F.chunk_offsets(wl)
    r = float(wl.schedule[-1])
    k = O.k_for_ratio(r, n_ctx, n_ctx)
    w = F.layer_weights(sh, 3)
    caches = [(prec.store(rng.standard_normal((offs[c + 1] - offs[c], sh.n_kv_heads, sh.head_dim)) * 0.3),
               prec.store(rng.standard_normal((offs[c + 1] - offs[c], sh.n_kv_heads, sh.head_dim)) * 0.3))
              for c in range(len(offs) - 1)]
    kept_ctx = np.sort(rng.choice(n_ctx, size=k, replace=False))

    def sample(frac):
        m = max(1, int(round(k * frac)))
        sel = np.concatenate([np.sort(rng.choice(kept_ctx, size=m, replace=False)), np.arange(n_ctx, n_tok)])
        hidden = rng.standard_normal((len(sel), sh.d_model))
        t0 = time.perf_counter()
        fk, fv = O.fuse_cache(sh, prec, caches, offs, n_q)
        res = O.blend_layer(sh, w, prec, hidden, fk, fv, n_ctx, sel, n_q, m / n_ctx)
        O.layer_rest(sh, w, prec, hidden, res["new_local"], res["out"])
        return time.perf_counter() - t0, len(sel)

    frac = 1.0 / 32
    runs = []
    spent = 0.0
    while True:
        t, rows = sample(frac)
        runs.append((frac, rows, t))
        spent += t
        if frac >= 1.0 or spent + 2.5 * t > budget_s:
            break
        frac = min(1.0, frac * 2)
    frac, rows, t = runs[-1]
    t_steady = t * (k + n_q) / rows
    f_steady = _oracle_layer_flops(sh, k + n_q, k + n_q, n_tok)
    t1 = t_steady * _oracle_layer_flops(sh, n_tok, n_tok, n_tok) / f_steady
    t2 = t_steady * _oracle_layer_flops(sh, n_tok, k + n_q, n_tok) / f_steady
    total = t1 + t2 + (sh.n_layers - 2) * t_steady
    out = {"value": round(n_ctx / total, 3), "unit": "context tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": (f"oracle (fp64 NumPy, bf16 rounding emulated): one steady layer of {wl.name} "
                      f"({k + n_q} kept rows over {n_tok} keys) run on {rows} of its kept rows in {t:.2f} s "
                      f"(runs: {[(round(a, 4), b, round(c, 2)) for a, b, c in runs]}); steady layer {t_steady:.1f} s "
                      f"by the row fraction, layers 1 and 2 {t1:.1f} s and {t2:.1f} s by the oracle's flop counts; "
                      f"blended prefill estimated at {total:.0f} s for {sh.n_layers} layers")}
    out.update(_host_info())
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="l70_16k", help="workload of the headline line (fixtures.CONFIGS)")
    ap.add_argument("--only-headline", action="store_true",
                    help="only the headline prompt's timed steps and kernel profile (profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="the headline workload only (with its overlap, HBM-resident and full-recompute passes), "
                         "no other configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--fetch", choices=("auto", "kernel", "copy"), default="auto",
                    help="how the headline engine fetches the cached KV (cb_set_fetch_mode): the library's choice "
                         "by chunk size, the fetch kernel reading pinned host memory over PCIe, or the copy engine "
                         "(one copy per chunk and K/V) + the position update")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device-to-device copy of 256 MiB, 3 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the fusion step is built and timed on a single MI355X "
              "(sharding across GPUs is a design note, not implemented)", file=sys.stderr)
        return 2
    import torch

    wl, head, other = run_headline(args)
    sh = wl.shape
    kernels = head.get("kernels", {})
    dom = max(kernels, key=lambda k: kernels[k]["ms_total_per_step"]) if kernels else None
    roofline = None
    if dom:
        dk = kernels[dom]
        roofline = {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"], "peak": dk["peak"],
                    "unit": dk["unit"], "frac": dk["frac"],
                    "traffic": traffic_from_profiles(dom, wl.name, dk["launches_per_step"]),
                    "mfma_busy_counter": mfma_busy_from_profiles(wl.name).get(dom),
                    "work_per_launch": dk["work_per_launch"], "us_per_launch": dk["us_per_launch"]}
    extra = {}
    if not args.only_headline and not args.no_extras:
        def guarded(fn, *a, **kw):
            try:
                return fn(*a, **kw)
            except Exception as e:  # an extra must not cost the headline line; the error is reported
                log(f"{fn.__name__} failed: {e!r}")
                return {"error": repr(e)}
        extra["qwen"] = guarded(run_qwen, args)
        extra["mistral_sweep"] = guarded(run_hbm_shape, "mistral_r15", (0.10, 0.15, 0.20), args)
        extra["yi"] = {"bf16": guarded(run_hbm_shape, "yi_r15", (0.15,), args),
                       "int8": guarded(run_hbm_shape, "yi_r15", (0.15,), args, int8=True)}
    if args.calib_copy:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        sync()
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(wl, args.cpu_budget)
        log(f"cpu oracle: {cpu['value']:.2f} context tokens/s on {cpu['cores']} threads")

    value = head["context_tokens_per_s"]
    busy = mfma_busy_from_profiles(wl.name)
    out = {
        "metric": "blended-prefill context tokens/s @ r=15% + per-layer ms; % HBM/MFMA peak",
        "value": value, "unit": "context tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["wall_ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sh.dtype, "data": "synthetic",
        "config": {"workload": describe(wl, "cached KV in pinned host memory (the chunk store's arena, filled by "
                                            "the chunk producer), fetched per layer two layers ahead on a copy "
                                            "stream inside every step; one prefill per step, T_blend from the "
                                            "first fetch enqueue to the last layer's end",
                                        "random weights N(0, 0.02) drawn on the device (torch generator, seeded)"),
                   "n_ctx": wl.n_ctx, "n_query": wl.n_query, "schedule": schedule_text(wl.schedule)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "t_blend_ms": head["t_blend_ms"],
        "per_layer_ms": head["per_layer_ms"],
        "kept_rows_per_layer": head["kept_rows_per_layer"],
        "kernels": {k: dict({kk: vv for kk, vv in v.items() if kk != "work_per_launch"},
                            **({"mfma_busy_counter": busy[k]} if k in busy else {})) for k, v in kernels.items()},
        "mfma_busy_counter": busy or None,
        "mfma_busy_note": ("mfma_busy_counter: share of SIMD cycles the MFMA pipe is busy over one step's launches "
                           "of each GEMM epilogue and of the attention (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / "
                           "(GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), profiles/mfma_busy_by_kernel_<workload>.txt; "
                           "gemm_kv_q holds the K/V and Q products, gemm_o_down the o- and down-projections); frac "
                           "is the event-timed rate against the 2.5 PFLOP/s peak at 2.4 GHz, so busy / frac ~ "
                           "2.4 GHz / the clock the chip holds"),
        "headline_detail": {k: v for k, v in head.items()
                            if k not in ("kernels", "t_blend_ms", "per_layer_ms", "kept_rows_per_layer")},
        "l70_4k": other,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
