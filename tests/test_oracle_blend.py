"""Pins of the oracle's fusion step against special cases the method reduces to.

* ratio 1 at every layer recomputes everything: fused KV and outputs equal an
  ordinary full prefill;
* one chunk at offset 0 is an exact prefix: for any schedule, the fused cache and
  the query outputs equal full prefill, and the deviation is zero;
* ratio 0 with one chunk at offset 0 reproduces the cache;
* chunk 0 of any prompt is a prefix: its rows never deviate;
* selected-set invariants of gradual filtering;
* the KV-size arithmetic printed on the LMCache page."""
import json
import os

import numpy as np
import pytest

import fixtures as F
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _setup(cfg):
    wl = F.get_config(cfg)
    sh = wl.shape
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    return wl, sh, W, F.embedding(sh)


@pytest.mark.parametrize("cfg", ["tiny3", "tiny_gqa"])
def test_ratio_one_is_full_prefill(cfg):
    wl, sh, W, E = _setup(cfg)
    r = O.blended_prefill(sh, W, E, F.chunk_tokens(wl), F.query_tokens(wl), [1.0] * sh.n_layers)
    full = O.full_prefill(sh, W, E, F.all_tokens(wl))
    for l, L in enumerate(r["layers"]):
        np.testing.assert_allclose(L["fused_k"], full["k"][l], atol=1e-12)
        np.testing.assert_allclose(L["fused_v"], full["v"][l], atol=1e-12)
        assert len(L["new_sel"]) == wl.n_tokens
    np.testing.assert_allclose(r["hidden"], full["hidden"][-1], atol=1e-12)


@pytest.mark.parametrize("sched", [(1.0, 0.3, 0.15), (1.0, 0.0, 0.0), (1.0, 0.5, 0.05), (0.2, 0.1, 0.1)])
def test_single_chunk_is_exact_prefix(sched):
    wl, sh, W, E = _setup("tiny3")
    chunk = F.chunk_tokens(wl)[0]
    q = F.query_tokens(wl)
    r = O.blended_prefill(sh, W, E, [chunk], q, list(sched))
    full = O.full_prefill(sh, W, E, np.concatenate([chunk, q]))
    n = len(chunk)
    for l, L in enumerate(r["layers"]):
        np.testing.assert_allclose(L["fused_k"], full["k"][l], atol=1e-12)
        np.testing.assert_allclose(L["fused_v"], full["v"][l], atol=1e-12)
        assert L["deviation"].max(initial=0.0) < 1e-20
    np.testing.assert_allclose(r["hidden"], full["hidden"][-1][r["sel"]], atol=1e-12)
    assert r["sel"][-len(q):].tolist() == list(range(n, n + len(q)))


def test_ratio_zero_single_chunk_reproduces_cache():
    wl, sh, W, E = _setup("tiny3")
    chunk = F.chunk_tokens(wl)[0]
    q = F.query_tokens(wl)
    caches = O.chunk_caches(sh, W, E, [chunk])
    r = O.blended_prefill(sh, W, E, [chunk], q, [1.0, 0.0, 0.0], caches=caches)
    n = len(chunk)
    for l, L in enumerate(r["layers"]):
        np.testing.assert_allclose(L["fused_k"][:n], caches[0][l][0], atol=1e-12)
        np.testing.assert_allclose(L["fused_v"][:n], caches[0][l][1], atol=1e-12)
    assert r["layers"][1]["new_sel"].tolist() == list(range(n, n + len(q)))  # query rows only
    assert r["layers"][2]["sel"].tolist() == list(range(n, n + len(q)))


@pytest.mark.parametrize("cfg", ["tiny3", "tiny_gqa"])
def test_chunk0_rows_never_deviate_and_set_invariants(cfg):
    wl, sh, W, E = _setup(cfg)
    r = O.blended_prefill(sh, W, E, F.chunk_tokens(wl), F.query_tokens(wl), wl.schedule)
    n0, n_ctx = wl.chunk_lens[0], wl.n_ctx
    qrows = np.arange(n_ctx, wl.n_tokens)
    for l, L in enumerate(r["layers"]):
        sel, new = L["sel"], L["new_sel"]
        cand = sel[sel < n_ctx]
        dev = L["deviation"]
        assert dev[cand < n0].max(initial=0.0) < 1e-20        # chunk 0 is an exact prefix
        if l > 0:
            assert dev[cand >= n0].max() > 1e-3               # later chunks do deviate
        assert np.all(np.diff(new) > 0)                       # ascending
        assert set(new.tolist()) <= set(sel.tolist())         # narrowing: S_{l+1} within S_l
        assert set(qrows.tolist()) <= set(new.tolist())       # query rows always kept
        k = O.k_for_ratio(wl.schedule[l], n_ctx, len(cand))
        assert len(new) == k + len(qrows)
        assert not np.isin(new, np.arange(n0)).any() or k > n_ctx - n0
    assert len(r["layers"][0]["new_sel"]) == wl.n_tokens      # layer 1 keeps every row


def test_error_shrinks_to_zero_at_full_recompute():
    """Qualitative trend of the explainer's quality table: more recompute, closer to full
    prefill; at 100% the fused result is exact."""
    wl, sh, W, E = _setup("tiny3")
    chunks, q = F.chunk_tokens(wl), F.query_tokens(wl)
    caches = O.chunk_caches(sh, W, E, chunks)
    full = O.full_prefill(sh, W, E, F.all_tokens(wl))
    qrows = np.arange(wl.n_ctx, wl.n_tokens)

    def err(r):
        res = O.blended_prefill(sh, W, E, chunks, q, [1.0, r, r], caches=caches)
        return np.abs(res["hidden"][-len(q):] - full["hidden"][-1][qrows]).max()

    e = {r: err(r) for r in (0.0, 0.15, 0.3, 1.0)}
    assert e[1.0] < 1e-12
    assert e[0.0] > e[0.3] > e[1.0]
    assert e[0.0] > e[0.15]


def test_kv_size_arithmetic_matches_printed_numbers():
    g = json.load(open(os.path.join(GOLDEN, "kv_sizes.json")))
    for case in g["per_token"]:
        shape = F.ModelShape(case["model"], case["layers"], 1, 1, case["kv_heads"], case["head_dim"],
                             1, 1, "bf16")
        assert O.cache_nbytes(shape, 1, case["elem_bytes"]) == case["bytes_per_token"]
    qs = F.get_config("qwen").shape
    ld = g["loaded"]
    assert ld["tokens"] == ld["chunks"] * ld["chunk_tokens"]
    gib = O.cache_nbytes(qs, ld["tokens"], 2) / 2 ** 30
    assert round(gib, 4) == ld["gib"]
    tr = g["transfer"]
    mb = O.cache_nbytes(qs, tr["tokens"], 2) / 1e6
    assert abs(mb - tr["approx_mb"]) < 1.0
    assert round(mb / tr["link_mb_per_s"], 1) == tr["approx_seconds"]
    be = O.cache_nbytes(qs, 1, 2) / (tr["prefill_ms_per_token"] * 1e-3) / 1e9
    assert round(be, 2) == tr["break_even_gb_per_s"]
    # the Qwen-shaped workload's host cache: 5,120 context tokens = exactly 140 MiB
    assert O.cache_nbytes(qs, 5120, 2) == 140 * 2 ** 20


def test_oracle_blocks_wrong_inputs():
    wl, sh, W, E = _setup("tiny")
    fk = np.zeros((wl.n_tokens, sh.n_kv_heads, sh.head_dim))
    h = np.zeros((3, sh.d_model)) + 0.1
    with pytest.raises(AssertionError):  # query rows missing from the selected set
        O.blend_layer(sh, W[0], O.F64, h, fk, fk, wl.n_ctx, [0, 1, 2], wl.n_query, 0.5)
