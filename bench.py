#!/usr/bin/env python3
"""Benchmark of the blended (CacheBlend-fused) prefill on one MI355X.

One step = one whole blended prefill of the Qwen2.5-1.5B-shaped workload: 28 decoder layers,
d_model 1536, 12 query / 2 KV heads of 128, FFN 8960, bf16, random-init weights N(0, 0.02);
10 independently cached chunks of 512 uniform-random tokens + a 64-token query; layer 1
recomputes every row, layer 2 keeps 30% of the context rows, layers 3.. keep 15%.
Per layer: RoPE position update of the cached K, RMSNorm + fresh K/V GEMM of the selected
rows, deviation + scatter, top-k, Q GEMM + sparse-query attention of the kept rows, then
o-projection and SwiGLU FFN on the kept rows.

value = context tokens / s = N_ctx * steps / wall time of the timed steps, with every input
(weights, chunk caches, token ids) resident in HBM when timing starts.  A step is replayed
from a HIP graph recorded once (the shapes of every layer are known on the host, so the
whole prefill is one graph); the eager-launch time of the same step is reported too.  The pinned-host
variant (cached KV fetched one layer ahead over PCIe on a second stream) is reported in
extra fields, not as value.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
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
DECODE_ROWS = 32           # fused-KV rows kept free after the prompt for the decode steps


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def schedule_text(sched):
    """'1.0, 0.30, 0.15 x 26' for a schedule whose last ratio repeats."""
    s = [float(x) for x in sched]
    head = s
    n_tail = 1
    while n_tail < len(s) and s[-n_tail - 1] == s[-1]:
        n_tail += 1
    head = s[: len(s) - n_tail]
    parts = [f"{x:.2f}" if x < 1 else "1.0" for x in head]
    tail = f"{s[-1]:.2f}" if s[-1] < 1 else "1.0"
    return ", ".join(parts + [tail + (f" x {n_tail}" if n_tail > 1 else "")])


def describe(wl):
    sh = wl.shape
    lens = sorted(set(wl.chunk_lens))
    chunks = (f"{len(wl.chunk_lens)}x{lens[0]}-token" if len(lens) == 1
              else f"{len(wl.chunk_lens)} ragged ({min(lens)}-{max(lens)} token)")
    return (f"{wl.name}: {sh.name}-shaped blended prefill, {sh.n_layers} layers, d_model {sh.d_model}, "
            f"{sh.n_q_heads}/{sh.n_kv_heads} heads of {sh.head_dim}, FFN {sh.ffn_dim}, {sh.dtype}; {chunks} cached "
            f"chunks + {wl.n_query}-token query, recompute {schedule_text(wl.schedule)}, cached KV resident in HBM")


def attention_flops(shape, records, n_query):
    """4 * H_q * d_h * sum over kept rows of (position + 1), summed over layers."""
    return [4.0 * shape.n_q_heads * shape.head_dim * float((r.new_sel.astype(np.int64) + 1).sum()) for r in records]


# The gate/up product's tile choice: (rows, cols, wavefronts, modelled microseconds per K-step
# of a workgroup) for each candidate; a launch costs ceil(workgroups / 256) K-step times, the
# cheapest candidate wins, and from 2,048 rows up the 256 x 256 tile is taken outright.
_SWIGLU_TILES = ((64, 128, 4, 0.72), (128, 128, 4, 0.83), (64, 256, 4, 1.04), (128, 256, 8, 1.13),
                 (256, 256, 8, 1.75), (128, 512, 8, 2.10))


def swiglu_tile(rows, n):
    """(bm, bn, wavefronts, workgroups) of the gate/up launch over `rows` rows and n = 2 ffn
    output columns, as the library plans it."""
    if rows >= 2048 and n % 256 == 0:
        bm, bn, nw = 256, 256, 8
    else:
        best = None
        for bm_, bn_, nw_, t in _SWIGLU_TILES:
            if n % bn_:
                continue
            cost = -(-(-(-rows // bm_) * (n // bn_)) // 256) * t
            if best is None or cost < best[0]:
                best = (cost, bm_, bn_, nw_)
        _, bm, bn, nw = best
    tiles = -(-rows // bm) * (n // bn)
    return bm, bn, nw, 8 * (-(-tiles // 8))  # workgroups: tiles rounded up to a multiple of 8


def gate_up_traffic(shape, kept_rows):
    """Mean HBM bytes per launch of the FFN gate/up GEMM over one step, from the committed
    rocprofv3 counter summary (FETCH_SIZE / WRITE_SIZE, scaled by a plain copy's reading),
    or None if that summary is missing, lacks one of the step's launches, or was taken on
    another version of the kernel source.  A launch is identified by its tile (in the kernel's
    name) and its grid size in threads (workgroups x 64 x wavefronts)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "gemm_gate_up_qwen_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256 (\S+): ([0-9a-f]{64})", text)
    if not m:
        return None
    src = os.path.join(ROOT, m.group(1))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != m.group(2):
        return None
    per_launch = {(int(bm), int(bn), int(g)): float(mb) for g, mb, bm, bn in re.findall(
        r"^\s*(\d+)\s+\d+\s+[\d.]+\s+[\d.]+\s+([\d.]+)\s+gemm_bf16_kernel<(\d+), (\d+),", text, re.M)}
    total = 0.0
    for rows in kept_rows:
        bm, bn, nw, wgs = swiglu_tile(rows, 2 * shape.ffn_dim)
        key = (bm, bn, wgs * 64 * nw)
        if key not in per_launch:
            return None
        total += per_launch[key] * 1e6
    return total / len(kept_rows)


def run_controller(eng, buf, tokens, offs, wl, fused, host, full_ms, overlap, steps):
    """The loading controller on this GPU, two ways, each followed by the pinned-host prefill run
    at the ratio it plans (layer 1 stays at 1):
      * cb_plan_ratio (the explainer's model): the load bandwidth of a whole step's cached KV
        fetched alone, and the full prefill split evenly over the layers and tokens;
      * cb_plan_ratio_measured: a layer's load time from the per-layer fetch measurement, and a
        layer's recompute time measured at ratio 1 (every row) and at ratio 0 (no context row:
        the fixed part), layer 1 counted at its own measured time.
    Both with a ratio floor of 5% (below the workload's 15%, so that the plan is not just the
    floor) and no ceiling."""
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
        for r in range(n + 2):
            if r == 2:
                eng.compute.synchronize()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, upload_inputs=False, **kw)
        eng.compute.synchronize()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e3

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
    t_first = float(t_full[0])
    t_full_l = float(np.median(t_full[1:]))
    t_fixed_l = min(float(np.median(t_zero[2:])), t_full_l)
    t_load_l = float(np.median(overlap["t_load_ms"])) * 1e-3
    meas = L.cb_plan_ratio_measured(nl, kv_layer, kv_layer / t_load_l, 0.0, t_first, t_full_l, t_fixed_l, r_min, r_max)
    meas_ms = run_plan(meas)
    log(f"controller (even split): load {bw / 1e9:.1f} GB/s, ratio {even.ratio:.3f}, predicted "
        f"{even.t_total * 1e3:.3f} ms, measured {even_ms:.3f} ms/step")
    log(f"controller (measured layer times: first {t_first * 1e3:.3f}, full {t_full_l * 1e3:.3f}, fixed "
        f"{t_fixed_l * 1e3:.3f}, load {t_load_l * 1e3:.3f} ms): ratio {meas.ratio:.3f} (load={meas.load}), "
        f"predicted {meas.t_total * 1e3:.3f} ms, measured {meas_ms:.3f} ms/step")
    return {"r_min": r_min, "r_max": r_max,
            "even_split": dict(summary(even, even_ms), load_bandwidth_GBps=round(bw / 1e9, 2),
                               prefill_us_per_token=round(pre * 1e6, 4)),
            "measured_layers": dict(summary(meas, meas_ms), t_first_ms=round(t_first * 1e3, 4),
                                    t_full_layer_ms=round(t_full_l * 1e3, 4),
                                    t_fixed_layer_ms=round(t_fixed_l * 1e3, 4)),
            "schedule": "1.0, then the planned ratio (pinned-host cache fetched two layers ahead; eager launches)"}


def _fetch_layer(eng, buf, host, offs, l, fused):
    from rag_kv_cache_amd import _lib as L
    n_chunks = len(offs) - 1
    L.cb_fetch_layer(eng.ctx, l, [int(host[l][c][0].data_ptr()) for c in range(n_chunks)],
                     [int(host[l][c][1].data_ptr()) for c in range(n_chunks)], offs, n_chunks,
                     int(buf.offsets.data_ptr()), int(fused[l][0].data_ptr()), int(fused[l][1].data_ptr()))


def run_overlap(eng, buf, tokens, offs, wl, fused, host, reps: int = 5, eps_ms: float = 0.02):
    """Per-layer T_load, T_recompute and T_overlapped of the pinned-host prefetched prefill, medians
    over `reps` runs:
      * T_load[l]: layer l's fetch alone (cached K/V of every chunk over PCIe + position update),
        HIP events around each launch on the copy stream, every layer fetched back to back with
        no compute running;
      * T_recompute[l]: layer l's compute alone (blend + rest), events on the compute stream, the
        fused buffers already holding the re-rotated cache (no fetch);
      * T_overlapped[l]: layer l on the compute stream in the pipelined run (fetches two layers
        ahead on the copy stream), including any wait for its fetch.
    The pipeline claim is checked per layer as T_overlapped <= max(T_load, T_recompute) + eps."""
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
    steady = list(range(3, nl))
    ok = [l for l in range(nl) if excess[l] <= eps_ms]
    log(f"overlap (steady medians): load {np.median([t_load[l] for l in steady]):.4f}, recompute "
        f"{np.median([t_rec[l] for l in steady]):.4f}, overlapped {np.median([t_ov[l] for l in steady]):.4f} ms; "
        f"{len(ok)}/{nl} layers within max(load, recompute) + {eps_ms} ms")
    r4 = lambda v: [round(x, 4) for x in v]
    return {"t_load_ms": r4(t_load), "t_recompute_ms": r4(t_rec), "t_overlapped_ms": r4(t_ov),
            "steady_median_ms": {"load": round(float(np.median([t_load[l] for l in steady])), 4),
                                 "recompute": round(float(np.median([t_rec[l] for l in steady])), 4),
                                 "overlapped": round(float(np.median([t_ov[l] for l in steady])), 4)},
            "sum_ms": {"load": round(sum(t_load), 4), "recompute": round(sum(t_rec), 4),
                       "overlapped": round(sum(t_ov), 4),
                       "max_per_layer": round(sum(max(a, b) for a, b in zip(t_load, t_rec)), 4)},
            "check": {"eps_ms": eps_ms, "layers_within": len(ok), "layers": nl,
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
    eng = Engine(sh, max_tokens=wl.n_tokens + 8)
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


def cpu_baseline(wl, budget_s: float = 25.0):
    """The oracle (fp64 NumPy with bf16 rounding points) on a bounded sample of the same
    workload: layer 1 (every row), layer 2 (all rows scored, 30% kept), layer 3 (15% kept)
    and steady layers until the time budget; tokens/s extrapolated to all layers.  The first
    steady layer is timed a second time with BLAS limited to one thread.  The chunk caches are
    random bf16-valued arrays of the real shape (their values do not change the oracle's cost);
    weights and tokens are the fixtures'."""
    import fixtures as F
    import oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    sh = wl.shape
    prec = O.Precision("bf16")
    rng = np.random.default_rng(0)
    E = F.embedding(sh)
    tokens = F.all_tokens(wl)
    n_ctx, n_tok, n_q = wl.n_ctx, wl.n_tokens, wl.n_query
    hidden = np.asarray(E[tokens], np.float64)
    del E
    sel = np.arange(n_tok)
    times = []
    single = None
    t_start = time.perf_counter()
    for l in range(sh.n_layers):
        w = F.layer_weights(sh, l + 1)
        kc = prec.store(rng.standard_normal((n_ctx, sh.n_kv_heads, sh.head_dim)) * 0.3)
        vc = prec.store(rng.standard_normal((n_ctx, sh.n_kv_heads, sh.head_dim)) * 0.3)

        def one_layer():
            fk, fv = O.fuse_cache(sh, prec, [(kc, vc)], [0, n_ctx], n_q)
            r = O.blend_layer(sh, w, prec, hidden, fk, fv, n_ctx, sel, n_q, wl.schedule[l])
            return O.layer_rest(sh, w, prec, hidden, r["new_local"], r["out"]), r["new_sel"]

        t0 = time.perf_counter()
        h_next, s_next = one_layer()
        times.append(time.perf_counter() - t0)
        if l == 3 and threadpool_limits is not None:
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                one_layer()
                single = time.perf_counter() - t0
        hidden, sel = h_next, s_next
        if l >= 4 and time.perf_counter() - t_start > budget_s:
            break
    steady = float(np.median(times[3:])) if len(times) > 3 else times[-1]
    total = sum(times[:3]) + steady * (sh.n_layers - 3)
    out = {"value": n_ctx / total, "unit": "context tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": (f"oracle (fp64 NumPy, bf16 rounding emulated) on layers 1-{len(times)} of the same workload "
                      f"with random-valued chunk caches of the real shape; layer times "
                      f"{[round(t, 3) for t in times]} s; blended prefill extrapolated as "
                      f"T1+T2+T3+{sh.n_layers - 3}*median(steady) = {total:.2f} s")}
    out.update(_host_info())
    if single is not None:
        out["single_thread_steady_layer_s"] = round(single, 3)
        out["all_threads_steady_layer_s"] = round(times[3], 3)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="qwen")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=25.0)
    ap.add_argument("--only-blend", action="store_true",
                    help="skip the pinned-host and full-recompute passes (profiling runs)")
    ap.add_argument("--ratios", default="",
                    help="comma-separated steady ratios: also time the graph-replayed prefill with the schedule "
                         "1.0, r, r, ... for each (e.g. 0.10,0.15,0.20 for the Mistral-7B-shaped sweep)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device-to-device copy of 256 MiB, 3 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the fusion step is built and timed on a single MI355X "
              "(sharding across GPUs is a design note, not implemented)", file=sys.stderr)
        return 2

    import torch
    import fixtures as F
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, capture_step, make_buffers, run_layers

    wl = F.get_config(args.config)
    sh = wl.shape
    chunks = F.chunk_tokens(wl)
    tokens = F.all_tokens(wl)
    offs = [int(o) for o in F.chunk_offsets(wl)]
    n_ctx, n_tok = wl.n_ctx, wl.n_tokens
    log(f"workload {wl.name}: {sh.n_layers} layers, d {sh.d_model}, heads {sh.n_q_heads}/{sh.n_kv_heads}, "
        f"N_ctx {n_ctx} + query {wl.n_query}")

    t0 = time.perf_counter()
    eng = Engine(sh, max_tokens=n_tok + 64)  # room for decode steps after the prefill
    for l in range(sh.n_layers):
        eng.load_layer(l, F.layer_weights(sh, l + 1))
    eng.load_embedding(F.embedding(sh))
    torch.cuda.synchronize()
    log(f"weights uploaded in {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    cache, host = build_chunk_caches(eng, chunks, pinned_host=True)
    log(f"chunk caches built in {time.perf_counter() - t0:.1f} s")

    extra = DECODE_ROWS  # rows after the prompt for the decode steps
    buf = make_buffers(eng, n_tok + extra, len(chunks))
    fused = [(eng.kv_empty(n_tok + extra), eng.kv_empty(n_tok + extra)) for _ in range(sh.n_layers)]
    cs = eng.compute
    rec = run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, cache=cache, record=True)
    attn_fl = attention_flops(sh, rec.records, wl.n_query)
    kept = [len(r.new_sel) for r in rec.records]

    def step(**kw):
        return run_layers(eng, buf, tokens, offs, wl.n_query, wl.schedule, fused, upload_inputs=False, **kw)

    for _ in range(args.warmup):
        step(cache=cache)
    cs.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(cache=cache)
    cs.synchronize()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / args.steps * 1e3
    log(f"blended prefill, eager launches: {eager_ms:.3f} ms/step")

    # the same step recorded once as a HIP graph and replayed: one launch per step
    graph = capture_step(eng, lambda: step(cache=cache))
    with torch.cuda.stream(cs):
        for _ in range(args.warmup):
            graph.replay()
    cs.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(cs):
        for _ in range(args.steps):
            graph.replay()
    cs.synchronize()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    ms_step = wall / args.steps * 1e3
    value = n_ctx * args.steps / wall
    log(f"blended prefill, graph replay: {ms_step:.3f} ms/step, {value:,.0f} context tokens/s")

    sweep = None
    if args.ratios:
        sweep = {}
        for r in [float(x) for x in args.ratios.split(",") if x]:
            sched = [1.0] + [r] * (sh.n_layers - 1)
            g = capture_step(eng, lambda: run_layers(eng, buf, tokens, offs, wl.n_query, sched, fused, cache=cache,
                                                     upload_inputs=False))
            with torch.cuda.stream(cs):
                for _ in range(args.warmup):
                    g.replay()
            cs.synchronize()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            with torch.cuda.stream(cs):
                for _ in range(args.steps):
                    g.replay()
            cs.synchronize()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) / args.steps * 1e3
            sweep[f"{r:.2f}"] = {"ms_per_step": round(ms, 4), "context_tokens_per_s": round(n_ctx / ms * 1e3, 1)}
            log(f"ratio {r:.2f}: {ms:.3f} ms/step, {n_ctx / ms * 1e3:,.0f} context tokens/s")
            del g

    # the same steps again with a HIP event pair around every launch (per-kernel durations)
    L.cb_profile_enable(eng.ctx, True)
    for _ in range(args.steps):
        step(cache=cache)
    cs.synchronize()
    L.cb_profile_enable(eng.ctx, False)

    kernels = {}
    for kid, name in enumerate(L.KERNEL_NAMES):
        ms, n, work = L.cb_profile_read(eng.ctx, kid)
        if n == 0:
            continue
        if kid == L.CB_K_ATTN:
            work = sum(attn_fl) * args.steps
        bound = "mfma" if kid in (L.CB_K_GEMM_KV, L.CB_K_GEMM_Q, L.CB_K_ATTN, L.CB_K_GEMM_O,
                                  L.CB_K_GEMM_GATE_UP, L.CB_K_GEMM_DOWN) else "hbm"
        rate = work / (ms * 1e-3) / (1e12 if bound == "mfma" else 1e9) if ms > 0 else 0.0
        peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
        kernels[name] = {"ms_total_per_step": round(ms / args.steps, 4), "launches_per_step": n // args.steps,
                         "us_per_launch": round(ms * 1e3 / n, 2), "bound": bound,
                         "achieved": round(rate, 2), "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                         "frac": round(rate / peak, 4)}
    dom = max(kernels, key=lambda k: kernels[k]["ms_total_per_step"])
    dk = kernels[dom]
    traffic = gate_up_traffic(sh, kept) if dom == "gemm_gate_up" and args.config == "qwen" else None
    roofline = {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"],
                "peak": PEAK_BF16_TFLOPS if dk["bound"] == "mfma" else PEAK_HBM_GBS, "unit": dk["unit"],
                "frac": dk["frac"], "traffic": None if traffic is None else round(traffic)}

    # per-layer latency (one extra profiled step with events at layer boundaries)
    evs = []
    step(cache=cache, layer_events=evs)
    cs.synchronize()
    per_layer = [evs[i].elapsed_time(evs[i + 1]) for i in range(len(evs) - 1)]

    pcie_ms = full_ms = controller = variants = decode_ms = store_res = overlap = reuse = peaks = int8 = None
    if not args.only_blend:
        # PCIe-inclusive variant: cached KV in pinned host memory, fetched one layer ahead
        for _ in range(2):
            step(host_cache=host)
        cs.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(host_cache=host)
        cs.synchronize()
        torch.cuda.synchronize()
        pcie_ms = (time.perf_counter() - t0) / args.steps * 1e3

        # full recompute on the same GPU and kernels (ratio 1 at every layer)
        full_sched = [1.0] * sh.n_layers
        run_layers(eng, buf, tokens, offs, wl.n_query, full_sched, fused, cache=cache, upload_inputs=False)
        cs.synchronize()
        t0 = time.perf_counter()
        n_full = max(3, args.steps // 4)
        for _ in range(n_full):
            run_layers(eng, buf, tokens, offs, wl.n_query, full_sched, fused, cache=cache, upload_inputs=False)
        cs.synchronize()
        full_ms = (time.perf_counter() - t0) / n_full * 1e3
        log(f"pinned-host prefetch: {pcie_ms:.3f} ms/step; full recompute: {full_ms:.3f} ms/step")
        overlap = run_overlap(eng, buf, tokens, offs, wl, fused, host)
        reuse = run_reuse(eng, buf, tokens, offs, wl, fused, cache, args.steps)
        controller = run_controller(eng, buf, tokens, offs, wl, fused, host, full_ms, overlap, args.steps)
        variants = run_variants(eng, buf, tokens, offs, wl, fused, cache, args.steps)
        decode_ms = run_decode(eng, buf, tokens, offs, wl, fused, cache)
        store_res = run_store(eng, buf, tokens, offs, wl, fused, args.steps)
        peaks = run_peaks(eng)
        int8 = run_int8(wl, args.steps, args.warmup) if wl.shape.dtype == "bf16" else None
    if args.calib_copy:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device=eng.device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(wl, args.cpu_budget)
        log(f"cpu oracle: {cpu['value']:.1f} context tokens/s on {cpu['cores']} threads")

    out = {
        "metric": "blended-prefill context tokens/s @ r=15% + per-layer ms; % HBM/MFMA peak",
        "value": round(value, 1), "unit": "context tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sh.dtype, "data": "synthetic",
        "config": {"workload": describe(wl), "n_ctx": n_ctx, "n_query": wl.n_query,
                   "schedule": schedule_text(wl.schedule)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_layer_ms": {"layer1": round(per_layer[0], 4), "layer2": round(per_layer[1], 4),
                         "layer3": round(per_layer[2], 4),
                         "steady_median": round(float(np.median(per_layer[3:])), 4)},
        "kept_rows_per_layer": kept[:4] + ["..."],
        "kernels": kernels,
        "pcie_prefetch": None if pcie_ms is None else {
            "ms_per_step": round(pcie_ms, 4), "context_tokens_per_s": round(n_ctx / pcie_ms * 1e3, 1),
            "host_kv_bytes_per_step": int(2 * sh.n_layers * n_ctx * sh.n_kv_heads * sh.head_dim * 2)},
        "prefetch_per_layer": overlap,
        "eager_ms_per_step": round(eager_ms, 4),
        "full_recompute_ms": None if full_ms is None else round(full_ms, 4),
        "full_reuse": reuse,
        "peaks_measured": peaks,
        "loading_controller": controller,
        "selection_variants": variants,
        "decode": decode_ms,
        "chunk_store": store_res,
        "ratio_sweep": sweep,
        "int8_weights": int8,
        "speedup_vs_full_recompute": None if full_ms is None else round(full_ms / ms_step, 3),
    }
    print(json.dumps(out), flush=True)
    eng.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
