"""Loading controller: how much to recompute given how fast the cache loads.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

From the pages:
* CacheBlend explainer, "Pipelined design": T_recompute = r * T_prefill and
  T_load = PerTokenKVSize * L / StorageThroughput (L read as the number of context tokens),
  overlapped so that the delay is max(T_recompute, T_load); section on threshold tuning: raise
  the recompute ratio on slow storage to hide the load, lower it on fast storage.
* CacheBlend review, "overlapping loading and recompute": per layer
  T_layer ~ max(T_load, T_recompute), plus filling and draining the pipeline.
* LMCache blog, section 5 (break-even): loading pays only if moving the KV is faster than
  recomputing it; per token, break-even bandwidth = KV bytes per token / prefill time per
  token (a fixed latency left aside); below it, recompute.

Readings: a layer's recompute time is linear in the ratio (the explainer's equation applied
per layer, T_prefill split evenly over the layers; plan_ratio_measured adds a measured
ratio-independent part and the full first layer); the planned ratio is the largest one whose
recompute still hides under the layer's load, kept inside [r_min, r_max] (the quality floor
and the point past which recompute cannot hide); when the bandwidth is at or below break-even
the plan is to recompute everything and load nothing.

Beyond the pages (plan_ratio_measured only; both terms default to zero, which is the model
above): the review's max(T_load, T_recompute) assumes the load and the recompute do not slow
each other; measured on one GPU the fetch of a later layer stretches the compute it runs
beside, by a measured `contention` (seconds of compute added per second of fetch running
beside it, and the same for the fetch when the compute runs beside it), so a layer takes
max(T_load, T_rec) + contention * min(T_load, T_rec); and the first filtering layer, which
scores every context row, costs a measured t_select over a later layer at the same ratio (the
review's "filling the pipeline").  The planned ratio stays the pages' rule (recompute as much
as the load hides).
"""
from __future__ import annotations

from dataclasses import dataclass


def t_load(n_tokens: int, kv_bytes_per_token: float, bandwidth: float, latency: float = 0.0) -> float:
    """Seconds to load the KV of n_tokens tokens (bytes per token over every layer covered)."""
    return n_tokens * kv_bytes_per_token / bandwidth + latency


def t_recompute(ratio: float, t_prefill: float) -> float:
    return ratio * t_prefill


def t_layer(t_load_layer: float, t_recompute_layer: float) -> float:
    return max(t_load_layer, t_recompute_layer)


def break_even_bandwidth(kv_bytes_per_token: float, prefill_s_per_token: float) -> float:
    """Bytes per second at which loading a token's KV costs exactly its prefill time."""
    return kv_bytes_per_token / prefill_s_per_token


@dataclass
class Plan:
    load: bool          # False: recompute every row, load nothing
    ratio: float        # recompute ratio of the blended layers (1.0 when not loading)
    t_load_layer: float
    t_recompute_layer: float
    t_layer: float
    t_total: float      # n_layers * t_layer: pipeline fill / drain left aside
    break_even: float


def plan_ratio(n_ctx: int, n_layers: int, kv_bytes_per_token_layer: float, bandwidth: float,
               prefill_s_per_token: float, r_min: float, r_max: float, latency_layer: float = 0.0) -> Plan:
    """The ratio to recompute per layer so that recompute hides under the layer's load."""
    t_pre_layer = n_ctx * prefill_s_per_token / n_layers  # full prefill time of one layer
    be = break_even_bandwidth(kv_bytes_per_token_layer * n_layers, prefill_s_per_token)
    tl = t_load(n_ctx, kv_bytes_per_token_layer, bandwidth, latency_layer)
    if bandwidth <= be:
        return Plan(False, 1.0, 0.0, t_pre_layer, t_pre_layer, n_layers * t_pre_layer, be)
    r = tl / t_pre_layer if t_pre_layer > 0 else r_max
    r = min(max(r, r_min), r_max)
    tr = t_recompute(r, t_pre_layer)
    return Plan(True, r, tl, tr, t_layer(tl, tr), n_layers * t_layer(tl, tr), be)


def plan_ratio_measured(n_layers: int, kv_bytes_layer: float, bandwidth: float, t_first_layer: float,
                        t_full_layer: float, t_fixed_layer: float, r_min: float, r_max: float,
                        latency_layer: float = 0.0, t_select_layer: float = 0.0,
                        contention: float = 0.0) -> Plan:
    """The same policy with a layer's recompute time measured on the GPU instead of an even
    split of the full prefill.  Reading: the explainer's T_recompute = r * T_prefill, taken per
    layer with a ratio-independent part added, T_recompute(r) = t_fixed + r (t_full - t_fixed)
    (t_full: a layer recomputing every row; t_fixed: a layer recomputing none, i.e. the query
    rows, norms, attention over the cache and the fixed kernel costs); t_fixed = 0 is the
    explainer's model.  With a load beside it a layer takes
    T_layer(r) = max(T_load, T_recompute(r)) + contention * min(T_load, T_recompute(r)): the
    longer of the two is stretched by the overlap with the other.  Loading pays when
    T_layer(r_min) < t_full (a layer that loads nothing recomputes every row with no fetch
    beside it).  The ratio is the largest in [r_min, r_max] whose recompute fits under the load,
    T_recompute(r) = T_load, as in plan_ratio.  The first
    layer recomputes every row whatever the plan (layer 1 scores all tokens), and when loading
    the next one, the first to filter, adds t_select: the step is
    t_first + t_select + (L - 1) T_layer.  break_even: the bandwidth at which a layer's load
    (latency aside) takes t_full."""
    be = kv_bytes_layer / t_full_layer
    tl = t_load(1, kv_bytes_layer, bandwidth, latency_layer)
    slope = t_full_layer - t_fixed_layer

    def rec(r):
        return t_fixed_layer + r * slope

    def layer(r):
        tr = rec(r)
        return max(tl, tr) + contention * min(tl, tr)

    if layer(r_min) >= t_full_layer:
        return Plan(False, 1.0, 0.0, t_full_layer, t_full_layer,
                    t_first_layer + (n_layers - 1) * t_full_layer, be)
    r = (tl - t_fixed_layer) / slope
    r = min(max(r, r_min), r_max)
    return Plan(True, r, tl, rec(r), layer(r), t_first_layer + t_select_layer + (n_layers - 1) * layer(r), be)
