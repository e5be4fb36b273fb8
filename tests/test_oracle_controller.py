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


def test_measured_plan_reduces_to_the_explainers_model():
    # t_fixed = 0 and the full prefill split evenly over the layers: the measured plan takes the
    # same decision, ratio and per-layer times as plan_ratio (pinned above to the pages' numbers);
    # only the total differs, by counting the first layer at its full cost
    rng = np.random.default_rng(4)
    for _ in range(300):
        n_ctx, L = int(rng.integers(64, 20000)), int(rng.integers(2, 90))
        kvb = float(rng.uniform(256, 40000))
        pre = float(10 ** rng.uniform(-6.5, -3.5))
        bw = float(10 ** rng.uniform(7, 12))
        r_min = float(rng.uniform(0, 0.3))
        r_max = float(rng.uniform(r_min, 1.0))
        a = C.plan_ratio(n_ctx, L, kvb, bw, pre, r_min, r_max)
        t_full = n_ctx * pre / L
        b = C.plan_ratio_measured(L, n_ctx * kvb, bw, t_full, t_full, 0.0, r_min, r_max)
        if abs(bw / a.break_even - 1) < 1e-9:
            continue                                   # the tie itself may go either way in rounding
        assert a.load == b.load
        assert abs(a.ratio - b.ratio) <= 1e-12 * max(1, a.ratio)
        for f in ("t_load_layer", "t_recompute_layer", "t_layer"):
            assert abs(getattr(a, f) - getattr(b, f)) <= 1e-12 * max(1e-9, getattr(a, f))
        assert abs(a.break_even / b.break_even - 1) < 1e-12
        assert abs(b.t_total - (t_full + (L - 1) * b.t_layer)) <= 1e-12 * b.t_total


def test_measured_plan_against_a_grid_search():
    # the largest ratio on a fine grid whose recompute still fits under the load
    rng = np.random.default_rng(5)
    grid = np.linspace(0.0, 1.0, 100001)
    for _ in range(200):
        t_full = float(rng.uniform(0.2e-3, 2e-3))
        t_fix = float(rng.uniform(0, 0.6)) * t_full
        tl = float(rng.uniform(0.3, 1.2)) * t_full
        r_min, r_max = 0.05, 0.8
        p = C.plan_ratio_measured(28, tl * 40e9, 40e9, 1e-3, t_full, t_fix, r_min, r_max)
        rec = t_fix + grid * (t_full - t_fix)
        if max(tl, t_fix + r_min * (t_full - t_fix)) >= t_full:
            assert not p.load and p.ratio == 1.0 and p.t_layer == t_full
            continue
        ok = grid[(rec <= tl) & (grid >= r_min) & (grid <= r_max)]
        want = ok.max() if len(ok) else r_min
        assert p.load and abs(p.ratio - want) <= 1.01e-5
        assert abs(p.t_load_layer - tl) <= 1e-12 * tl
        assert p.t_layer == max(p.t_load_layer, p.t_recompute_layer)
        assert abs(p.t_total - (1e-3 + 27 * p.t_layer)) <= 1e-15 + 1e-12 * p.t_total


def test_measured_plan_special_cases():
    # a fixed recompute cost above the load: nothing more can hide, the ratio floor is used
    p = C.plan_ratio_measured(10, 1e6, 1e10, 2e-3, 1e-3, 0.5e-3, 0.1, 0.9)   # load 0.1 ms
    assert p.load and p.ratio == 0.1 and abs(p.t_layer - (0.5e-3 + 0.1 * 0.5e-3)) < 1e-15
    # load slower than recomputing the layer: recompute everything
    p = C.plan_ratio_measured(10, 1e6, 0.5e9, 2e-3, 1e-3, 0.2e-3, 0.1, 0.9)  # load 2 ms
    assert not p.load and p.ratio == 1.0 and abs(p.t_total - (2e-3 + 9e-3)) < 1e-15
    # the review's Llama-7B example (load 16 ms against 3 ms of recompute): load-bound, the plan
    # raises the ratio to its ceiling and the layer takes the load time
    p = C.plan_ratio_measured(32, 16e-3 * 1e9, 1e9, 20e-3, 20e-3, 0.0, 0.15, 0.5)
    assert p.load and p.ratio == 0.5 and abs(p.t_layer - 16e-3) < 1e-15


def test_contended_plan_against_a_grid_search():
    # with contention k a loading layer takes max(T_load, T_rec) + k min(T_load, T_rec); the ratio
    # is still the largest on a fine grid whose recompute fits under the load (else r_min), and
    # the plan loads only when that layer time at r_min beats recomputing the layer
    rng = np.random.default_rng(11)
    grid = np.linspace(0.0, 1.0, 100001)
    for _ in range(200):
        t_full = float(rng.uniform(0.2e-3, 2e-3))
        t_fix = float(rng.uniform(0, 0.6)) * t_full
        tl = float(rng.uniform(0.3, 1.2)) * t_full
        k = float(rng.uniform(0.0, 0.5))
        t_sel = float(rng.uniform(0.0, 0.3)) * t_full
        r_min, r_max = 0.05, 0.8
        p = C.plan_ratio_measured(28, tl * 40e9, 40e9, 1e-3, t_full, t_fix, r_min, r_max,
                                  t_select_layer=t_sel, contention=k)
        rec = t_fix + grid * (t_full - t_fix)
        tr_min = t_fix + r_min * (t_full - t_fix)
        if max(tl, tr_min) + k * min(tl, tr_min) >= t_full:
            assert not p.load and p.ratio == 1.0 and p.t_layer == t_full
            assert abs(p.t_total - (1e-3 + 27 * t_full)) <= 1e-12 * p.t_total
            continue
        ok = grid[(rec <= tl) & (grid >= r_min) & (grid <= r_max)]
        want = ok.max() if len(ok) else r_min
        assert p.load and abs(p.ratio - want) <= 1.01e-5
        tr = t_fix + p.ratio * (t_full - t_fix)
        assert abs(p.t_layer - (max(tl, tr) + k * min(tl, tr))) <= 1e-15 + 1e-12 * p.t_layer
        assert abs(p.t_total - (1e-3 + t_sel + 27 * p.t_layer)) <= 1e-15 + 1e-12 * p.t_total


def test_contended_plan_worked_cases():
    # hand-worked: load 1 ms, t_fixed 0.2 ms, t_full 2.2 ms (slope 2 ms), contention 0.25:
    # r = (1 - 0.2) / 2 = 0.4, T_rec = 1 ms, T_layer = max(1, 1) + 0.25 * 1 = 1.25 ms;
    # 10 layers, first 3 ms, first filter +0.5 ms: 3 + 0.5 + 9 * 1.25 = 14.75 ms
    p = C.plan_ratio_measured(10, 1e6, 1e9, 3e-3, 2.2e-3, 0.2e-3, 0.05, 0.9, t_select_layer=0.5e-3, contention=0.25)
    assert p.load and abs(p.ratio - 0.4) < 1e-12 and abs(p.t_layer - 1.25e-3) < 1e-15
    assert abs(p.t_total - 14.75e-3) < 1e-15
    # a light load under the ratio floor 0.5: T_rec = 1.2 ms, T_layer = 1.2 + 0.25 * 0.1 = 1.225 ms
    p = C.plan_ratio_measured(10, 1e5, 1e9, 3e-3, 2.2e-3, 0.2e-3, 0.5, 0.9, contention=0.25)
    assert p.load and p.ratio == 0.5 and abs(p.t_layer - 1.225e-3) < 1e-15
    # contention that makes the floor's layer slower than recomputing: floor 0.9 -> T_rec 2.0 ms,
    # T_layer = 2.0 + 0.5 * 1.0 = 2.5 ms >= 2.2 ms: recompute everything, no first-filter cost
    p = C.plan_ratio_measured(10, 1e6, 1e9, 3e-3, 2.2e-3, 0.2e-3, 0.9, 1.0, t_select_layer=0.5e-3, contention=0.5)
    assert not p.load and p.ratio == 1.0 and abs(p.t_total - (3e-3 + 9 * 2.2e-3)) < 1e-15
    # the same without contention loads (T_layer = max(1, 2.0) = 2.0 < 2.2)
    p = C.plan_ratio_measured(10, 1e6, 1e9, 3e-3, 2.2e-3, 0.2e-3, 0.9, 1.0)
    assert p.load and p.ratio == 0.9 and abs(p.t_layer - 2.0e-3) < 1e-15
