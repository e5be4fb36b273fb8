"""Pins of the oracle's loading controller against the numbers the pages print (break-even
bandwidths, a slow link losing to recompute, per-layer load vs recompute examples) and
against the explainer's qualitative rule (faster storage, lower ratio)."""
import json
import os

import numpy as np
import pytest

from oracle import controller as C

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "controller_examples.json")))


def test_break_even_of_the_qwen_example():
    g = G["lmcache_s5"]
    per_tok = g["prefill_ms"] * 1e-3 / g["tokens"]
    be = C.break_even_bandwidth(g["kv_bytes_per_token"], per_tok)
    assert abs(be / 1e9 - g["printed_break_even_GBps"]) < 0.005
    # CPU memory is more than 50x faster than break-even
    assert g["cpu_memory_GBps"] * 1e9 / be > g["printed_cpu_over_break_even_at_least"]


def test_slow_link_loses_to_recompute():
    g = G["lmcache_s5"]
    kv = g["tokens"] * g["kv_bytes_per_token"]
    assert abs(kv / 1e6 - g["kv_MB_printed"]) < 1.0
    tl = C.t_load(g["tokens"], g["kv_bytes_per_token"], g["link_MBps"] * 1e6)
    assert abs(tl - g["printed_link_load_s"]) < 0.05
    assert tl > g["printed_recompute_s"]
    # the plan at that bandwidth recomputes everything (28 layers, bytes per layer)
    p = C.plan_ratio(g["tokens"], 28, g["kv_bytes_per_token"] / 28, g["link_MBps"] * 1e6,
                     g["prefill_ms"] * 1e-3 / g["tokens"], 0.05, 0.5)
    assert not p.load and p.ratio == 1.0


@pytest.mark.parametrize("case", G["lmcache_s9_6"]["cases"])
def test_break_even_of_the_8b_example(case):
    be = C.break_even_bandwidth(G["lmcache_s9_6"]["kv_bytes_per_token"], case["prefill_ms_per_token"] * 1e-3)
    assert abs(be / 1e9 - case["printed_break_even_GBps"]) < 0.06


def test_disk_margin_over_break_even():
    g = G["lmcache_s9_6"]
    be = C.break_even_bandwidth(g["kv_bytes_per_token"], g["cases"][1]["prefill_ms_per_token"] * 1e-3)
    assert abs(g["disk_GBps"] * 1e9 / be - g["printed_disk_over_break_even"]) < 0.7


@pytest.mark.parametrize("ex", G["review_overlap"])
def test_layer_time_is_the_larger_of_load_and_recompute(ex):
    t = C.t_layer(ex["load_ms"], ex["recompute_ms"])
    assert t == max(ex["load_ms"], ex["recompute_ms"])
    assert (ex["load_ms"] > ex["recompute_ms"]) == (ex["bound"] == "load")


def test_plan_hides_recompute_under_load_and_falls_with_bandwidth():
    n_ctx, L, per_tok_layer = 5120, 28, 1024.0      # Qwen2.5-1.5B-shaped, bf16
    pre = 20e-3 / 5184                               # seconds per token of full prefill
    be = C.break_even_bandwidth(per_tok_layer * L, pre)
    # at or below break-even: recompute everything (a faster GPU raises break-even)
    for bw in (0.5 * be, be):
        p = C.plan_ratio(n_ctx, L, per_tok_layer, bw, pre, 0.05, 0.6)
        assert not p.load and p.ratio == 1.0
    ratios = []
    for bw in np.geomspace(1.01 * be, 1e3 * be, 25):
        p = C.plan_ratio(n_ctx, L, per_tok_layer, bw, pre, 0.05, 0.6)
        assert p.load
        assert 0.05 <= p.ratio <= 0.6
        if 0.05 < p.ratio < 0.6:                     # not clamped: recompute exactly hidden
            assert abs(p.t_recompute_layer - p.t_load_layer) <= 1e-12 + 1e-9 * p.t_load_layer
        assert p.t_layer == max(p.t_load_layer, p.t_recompute_layer)
        ratios.append(p.ratio)
    assert all(a >= b for a, b in zip(ratios, ratios[1:]))   # faster storage, lower ratio
    assert ratios[0] == 0.6 and ratios[-1] == 0.05
    # unclamped, the ratio is the load / prefill time ratio of a layer: at 10x break-even, 0.1
    p = C.plan_ratio(n_ctx, L, per_tok_layer, 10 * be, pre, 0.01, 1.0)
    assert abs(p.ratio - 0.1) < 1e-12
