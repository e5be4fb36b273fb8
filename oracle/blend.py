"""The fusion step itself: deviation, gradual filtering, scatter, sparse-query attention.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Per layer l with selected row set S_l (ascending absolute positions, always holding
every query row), following the per-layer flow of the CacheBlend review and the
"HKVD token selection" / "Gradual filtering" sections of the CacheBlend explainer:

  1. x = RMSNorm(h[S_l]); fresh Q, K, V of S_l; RoPE at the rows' true positions.
  2. deviation d_j = ||K_new[j] - K_fused[j]||^2 + ||V_new[j] - V_fused[j]||^2 for the
     context rows of S_l, against the re-rotated cache of this layer before it is
     updated.  The pages define the deviation as an L2 norm of the KV difference; the
     squared norm ranks identically and is what is reported.  KV_full of the page's
     equation is not available without a full prefill, so the fresh KV of the current
     partially fused inputs stands in for it (the review: later layers compare the
     recomputed KV of earlier candidates with the stored KV).
  3. k_l = floor(r_l * N_ctx + 1/2) clamped to the candidates available (ratios count
     context tokens; query rows are always kept and not counted).
  4. T = top-k_l by (d descending, position ascending); the decision is taken on the
     float32 rounding of d, the precision the GPU ranks in.
  5. S_{l+1} = T u query rows, ascending.
  6. fused[S_l] <- fresh K, V (every recomputed row, including rows dropped in 4).
  7. attention output for the rows of S_{l+1} over fused rows 0..p (causal).
  8. rest of the layer (o-projection, residual, FFN) on the rows of S_{l+1}.
Layer 1 runs at ratio 1 (every row recomputed): at layer 1 a token's KV depends only on
its own embedding and position, so its deviation is rounding noise and ranking it would
select arbitrary rows.  The configured ratios apply from layer 2 on.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

from .model import (F64, Precision, causal_attention, chunk_caches, mlp, project, rmsnorm,
                    rope_delta, rope_rotate)


def k_for_ratio(ratio: float, n_ctx: int, n_avail: int) -> int:
    """Number of context rows kept: floor(r * N_ctx + 1/2) with r taken as float32,
    clamped to [0, n_avail]."""
    k = math.floor(float(np.float32(ratio)) * n_ctx + 0.5)
    return max(0, min(int(k), int(n_avail)))


def topk_select(d: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of d, ties broken by lower index, returned ascending.
    d is compared as float32 values."""
    d32 = np.asarray(d).astype(np.float32)
    idx = np.arange(len(d32))
    order = np.lexsort((idx, -d32.astype(np.float64)))
    return np.sort(order[:k])


def kv_deviation(k_new, v_new, k_old, v_old) -> np.ndarray:
    """Per-row squared L2 distance over all K and V elements of the layer ([n, H_kv, d_h] each)."""
    dk = np.asarray(k_new, np.float64) - np.asarray(k_old, np.float64)
    dv = np.asarray(v_new, np.float64) - np.asarray(v_old, np.float64)
    return (dk * dk).sum(axis=(1, 2)) + (dv * dv).sum(axis=(1, 2))


def cosine_deviation(k_new, v_new, k_old, v_old) -> np.ndarray:
    """Per-row cosine deviation 1 - <a, b> / (|a| |b|), with a and b the row's fresh and cached
    K and V concatenated over every KV head ([n, H_kv, d_h] each).  The KVBoost page
    (section on seam repair, deviation-guided strategy) ranks tokens by the deviation of the
    token-wise cosine similarity between cached and recomputed KV; the vector compared is the
    same K|V row the L2 score uses (reading).  A zero vector has no direction: the deviation
    is 0 when both rows are zero and 1 when only one is (reading)."""
    a = np.concatenate([np.asarray(k_new, np.float64).reshape(len(k_new), -1),
                        np.asarray(v_new, np.float64).reshape(len(v_new), -1)], axis=1)
    b = np.concatenate([np.asarray(k_old, np.float64).reshape(len(k_old), -1),
                        np.asarray(v_old, np.float64).reshape(len(v_old), -1)], axis=1)
    dot = (a * b).sum(axis=1)
    na = (a * a).sum(axis=1)
    nb = (b * b).sum(axis=1)
    out = np.empty(len(a))
    for i in range(len(a)):
        if na[i] == 0.0 or nb[i] == 0.0:
            out[i] = 0.0 if na[i] == nb[i] else 1.0
        else:
            out[i] = 1.0 - dot[i] / math.sqrt(na[i] * nb[i])
    return out


def seam_positions(chunk_offsets: Sequence[int], n_query: int, window: int) -> np.ndarray:
    """The spatial seam-repair set of the KVBoost page (section on seam repair, spatial
    strategy): the `window` positions just before every chunk boundary (default 16 on the
    page), re-encoded with the whole context, plus every query row; ascending.  The boundary
    after the last chunk is the one with the query (reading: every chunk has a boundary
    after it); a window longer than its chunk covers the whole chunk."""
    offs = [int(o) for o in chunk_offsets]
    pos = []
    for c in range(len(offs) - 1):
        lo, hi = offs[c], offs[c + 1]
        pos.extend(range(max(lo, hi - int(window)), hi))
    n_ctx = offs[-1]
    pos.extend(range(n_ctx, n_ctx + int(n_query)))
    return np.asarray(pos, dtype=np.int64)


def fuse_cache(shape, prec: Precision, layer_cache: Sequence, chunk_offsets: Sequence[int],
               n_query: int):
    """Fused K/V buffers of one layer before any recompute: chunk c's cached K rotated by
    R(o_c), its V copied, at rows [o_c, o_{c+1}); query rows zero.  [N, H_kv, d_h] each."""
    offs = np.asarray(chunk_offsets)
    n_ctx = int(offs[-1])
    hkv, dh = shape.n_kv_heads, shape.head_dim
    fk = np.zeros((n_ctx + n_query, hkv, dh))
    fv = np.zeros((n_ctx + n_query, hkv, dh))
    if n_ctx:
        kc = np.concatenate([np.asarray(k, np.float64) for k, _ in layer_cache])
        vc = np.concatenate([np.asarray(v, np.float64) for _, v in layer_cache])
        fk[:n_ctx] = prec.store(rope_delta(kc, offs, shape.rope_base))
        fv[:n_ctx] = vc
    return fk, fv


def blend_layer(shape, w: Dict[str, np.ndarray], prec: Precision, hidden_sel: np.ndarray,
                fused_k: np.ndarray, fused_v: np.ndarray, n_ctx: int, sel_idx: Sequence[int],
                n_query: int, ratio: float, new_sel_override: Optional[Sequence[int]] = None,
                score: str = "l2"):
    """Steps 1-7 above for one layer.  fused_k / fused_v are not modified; updated copies are
    returned.  `new_sel_override` replaces the selected set (used to evaluate attention on a
    set chosen elsewhere, e.g. when a near-tie was resolved the other way).  score "l2" is
    step 2's deviation, "cosine" the KVBoost variant (cosine_deviation)."""
    hq, hkv, dh = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    sel = np.asarray(sel_idx, dtype=np.int64)
    n_sel = len(sel)
    n_tok = fused_k.shape[0]
    assert n_tok == n_ctx + n_query and n_sel >= n_query
    assert np.all(np.diff(sel) > 0), "sel_idx must be strictly ascending"
    assert np.array_equal(sel[n_sel - n_query:], np.arange(n_ctx, n_tok)), "query rows must be selected"
    n_cand = n_sel - n_query

    x = prec.store(rmsnorm(hidden_sel, w["g_attn"], shape.rms_eps))
    k_new = prec.store(rope_rotate(project(x, w["w_k"]).reshape(n_sel, hkv, dh), sel, shape.rope_base))
    v_new = prec.store(project(x, w["w_v"]).reshape(n_sel, hkv, dh))

    dev_fn = {"l2": kv_deviation, "cosine": cosine_deviation}[score]
    dev = dev_fn(k_new[:n_cand], v_new[:n_cand], fused_k[sel[:n_cand]], fused_v[sel[:n_cand]])
    k = k_for_ratio(ratio, n_ctx, n_cand)
    keep = topk_select(dev, k)
    new_local = np.concatenate([keep, np.arange(n_cand, n_sel)]).astype(np.int64)
    if new_sel_override is not None:
        pos_to_local = {int(p): i for i, p in enumerate(sel)}
        new_local = np.array([pos_to_local[int(p)] for p in new_sel_override], dtype=np.int64)
    new_sel = sel[new_local]

    fk = fused_k.copy()
    fv = fused_v.copy()
    fk[sel] = k_new
    fv[sel] = v_new

    xq = x[new_local]
    q = prec.store(rope_rotate(project(xq, w["w_q"]).reshape(len(new_local), hq, dh), new_sel,
                               shape.rope_base))
    out = prec.store(causal_attention(q, fk, fv, new_sel)).reshape(len(new_local), hq * dh)
    return {"fused_k": fk, "fused_v": fv, "k_new": k_new, "v_new": v_new, "deviation": dev,
            "k": k, "new_sel": new_sel, "new_local": new_local, "q": q, "out": out}


def attn_residual(w: Dict[str, np.ndarray], hidden_sel: np.ndarray, new_local: Sequence[int],
                  out: np.ndarray) -> np.ndarray:
    """First half of step 8: h1 = h[kept] + out W_o^T (the residual after attention)."""
    return np.asarray(hidden_sel, np.float64)[np.asarray(new_local)] + project(out, w["w_o"])


def layer_rest(shape, w: Dict[str, np.ndarray], prec: Precision, hidden_sel: np.ndarray,
               new_local: Sequence[int], out: np.ndarray) -> np.ndarray:
    """Step 8: o-projection plus residual on the kept rows, then the SwiGLU FFN block.
    Returns the residual-stream rows of S_{l+1} for the next layer."""
    h1 = attn_residual(w, hidden_sel, new_local, out)
    return mlp(h1, w, shape.rms_eps, prec)


def blended_prefill(shape, weights: List[Dict[str, np.ndarray]], emb: np.ndarray,
                    chunks: Sequence[np.ndarray], query: np.ndarray, schedule: Sequence[float],
                    prec: Precision = F64, caches=None, score: str = "l2",
                    initial_sel: Optional[Sequence[int]] = None):
    """The whole fused prefill: per-chunk caches, then per layer fuse -> blend -> rest.
    initial_sel: the rows recomputed at layer 1 (default every row; seam_positions gives the
    spatial seam-repair set, kept at every layer with ratio 1).
    Returns dict(layers=[per-layer blend_layer results + 'sel'], hidden=final rows,
    sel=final selected set, caches=the chunk caches)."""
    if caches is None:
        caches = chunk_caches(shape, weights, emb, chunks, prec)
    offs = np.concatenate([[0], np.cumsum([len(c) for c in chunks])]).astype(np.int64)
    n_ctx = int(offs[-1])
    n_query = len(query)
    tokens = np.concatenate(list(chunks) + [np.asarray(query)]).astype(np.int64)
    n_tok = len(tokens)
    assert len(schedule) == len(weights)
    sel = np.arange(n_tok) if initial_sel is None else np.asarray(initial_sel, np.int64)
    hidden = np.asarray(emb[tokens[sel]], np.float64)
    layers = []
    for li, w in enumerate(weights):
        fk, fv = fuse_cache(shape, prec, [c[li] for c in caches], offs, n_query)
        r = blend_layer(shape, w, prec, hidden, fk, fv, n_ctx, sel, n_query, schedule[li], score=score)
        r["sel"] = sel
        r["hidden_in"] = hidden
        hidden = layer_rest(shape, w, prec, hidden, r["new_local"], r["out"])
        r["hidden_out"] = hidden
        layers.append(r)
        sel = r["new_sel"]
    return {"layers": layers, "hidden": hidden, "sel": sel, "caches": caches, "offsets": offs}


def decode_step(shape, weights: List[Dict[str, np.ndarray]], emb: np.ndarray, prec: Precision,
                fused: Sequence, n_past: int, tokens: Sequence[int]):
    """Generation with the fused KV (CacheBlend review: generate with the fused KV cache after
    the blended prefill): the n_new = len(tokens) new tokens at positions n_past .. get fresh
    Q/K/V at every layer, their K/V are appended to the layer's fused KV (rows n_past ..), and
    they attend causally to every fused row up to their position.  This is step 1-8 above with
    every past row as (already fused) context, the new rows as query rows and nothing to rank.
    fused[l] = (K, V) [n_past, H_kv, d_h]; returns the extended fused KV per layer, the new
    rows' hidden state after the last layer and each layer's attention output."""
    toks = np.asarray(tokens, np.int64)
    n_new = len(toks)
    sel = np.arange(n_past, n_past + n_new)
    hidden = np.asarray(emb[toks], np.float64)
    out_fused, outs = [], []
    for li, w in enumerate(weights):
        k0, v0 = fused[li]
        fk = np.concatenate([np.asarray(k0, np.float64)[:n_past], np.zeros((n_new,) + k0.shape[1:])])
        fv = np.concatenate([np.asarray(v0, np.float64)[:n_past], np.zeros((n_new,) + v0.shape[1:])])
        r = blend_layer(shape, w, prec, hidden, fk, fv, n_past, sel, n_new, 0.0)
        hidden = layer_rest(shape, w, prec, hidden, r["new_local"], r["out"])
        out_fused.append((r["fused_k"], r["fused_v"]))
        outs.append(r["out"])
    return {"fused": out_fused, "hidden": hidden, "out": outs}
