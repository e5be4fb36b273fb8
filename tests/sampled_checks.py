"""Sampled, teacher-forced checks of one layer of a large blended prefill against the oracle.

At sizes the oracle cannot run whole, each sampled layer is checked with the GPU's own inputs
of that layer (the residual rows entering it and the fused cache it attends over):
  * the kept set is exactly the top-k of the GPU's deviations (float32, ties to the lower
    position) and ends with every query row;
  * the deviation of sampled candidate rows equals the oracle's (fresh K/V against the
    re-rotated GPU cache row);
  * sampled recomputed rows of the fused cache hold the oracle's fresh K/V, sampled rows that
    were not recomputed hold the re-rotated chunk cache (V bit for bit);
  * the attention output and the layer output of sampled kept rows (always some query rows);
and a decode step on the fused KV is checked layer by layer the same way.
"""
from __future__ import annotations

import numpy as np

import fixtures as F
import oracle as O
from parity_util import assert_close, ffn_tol_scale


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_layer(wl, layer, w, rec, h, cache_kv, fused_kv, n_sample=24, seed=100):
    """wl: the workload; layer: 0-based; w: the oracle's weights of that layer; rec: the GPU's
    LayerRecord; h: [len(rec.sel), d] residual rows entering the layer (GPU values);
    cache_kv / fused_kv: (K, V) device tensors of the chunk cache and fused cache of the layer."""
    sh = wl.shape
    prec = O.Precision("bf16")
    sel, new = rec.sel, rec.new_sel
    n_ctx, n_q = wl.n_ctx, wl.n_query
    n_cand = len(sel) - n_q
    k = O.k_for_ratio(wl.schedule[layer], n_ctx, n_cand)
    offs = F.chunk_offsets(wl)
    rng = np.random.default_rng(seed + layer)
    hq, hkv, dh = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    assert h.shape[0] == len(sel)

    # 1. kept set
    dev = rec.deviation.astype(np.float32)
    assert len(new) == k + n_q
    assert np.array_equal(new[k:], np.arange(n_ctx, n_ctx + n_q))
    assert np.array_equal(new[:k], np.sort(sel[:n_cand][O.topk_select(dev, k)]))

    # 2. deviation of sampled candidate rows
    ck, cv = to_np(cache_kv[0]), to_np(cache_kv[1])
    rows = rng.choice(n_cand, size=min(n_sample, n_cand), replace=False)
    pos = sel[rows]
    chunk_of = np.searchsorted(offs, pos, side="right") - 1
    k_rot = prec.store(O.rope_rotate(ck[pos], offs[chunk_of], sh.rope_base))
    x = prec.store(O.rmsnorm(h[rows], w["g_attn"], sh.rms_eps))
    k_new = prec.store(O.rope_rotate(O.project(x, w["w_k"]).reshape(-1, hkv, dh), pos, sh.rope_base))
    v_new = prec.store(O.project(x, w["w_v"]).reshape(-1, hkv, dh))
    fk, fv = to_np(fused_kv[0]), to_np(fused_kv[1])
    # 2a. the score's arithmetic on the GPU's own fresh rows (scattered into the fused cache)
    d_own = O.kv_deviation(fk[pos], fv[pos], k_rot, cv[pos])
    err = np.abs(dev[rows] - d_own) - 1e-3 * d_own
    assert err.max() <= 1e-3, f"layer {layer + 1}: deviation of the GPU's fresh rows, err {err.max():.3e}"
    # 2b. against the oracle's fresh rows: each stored bf16 element of either side may sit one
    # rounding step (at most 2^-7 |x|) away from the other side's, so per element the squared
    # difference moves by at most e (2 |delta| + e) with e the two steps' sum
    d_ref = O.kv_deviation(k_new, v_new, k_rot, cv[pos])
    slack = np.zeros(len(rows))
    for a, b in ((k_new, k_rot), (v_new, cv[pos])):
        e = 2.0 ** -7 * (np.abs(a) + np.abs(b))
        slack += (e * (2 * np.abs(a - b) + e)).sum(axis=(1, 2))
    err = np.abs(dev[rows] - d_ref) - 1e-3 * d_ref - slack
    assert err.max() <= 1e-3, f"layer {layer + 1}: deviation err {err.max():.3e} beyond the rounding bound"

    # 3. fused cache
    assert_close(fk[pos], k_new, "bf16", f"layer {layer + 1}: fused K of recomputed rows")
    assert_close(fv[pos], v_new, "bf16", f"layer {layer + 1}: fused V of recomputed rows")
    untouched = np.setdiff1d(np.arange(n_ctx), sel)
    if len(untouched):
        urows = rng.choice(untouched, size=min(n_sample, len(untouched)), replace=False)
        uchunk = np.searchsorted(offs, urows, side="right") - 1
        rot = prec.store(O.rope_rotate(ck[urows], offs[uchunk], sh.rope_base))
        assert_close(fk[urows], rot, "bf16", f"layer {layer + 1}: re-rotated K of untouched rows")
        assert np.array_equal(fv[urows], cv[urows])

    # 4. attention output and layer output of sampled kept rows
    loc = {int(p): i for i, p in enumerate(sel)}
    tail = min(8, len(new))
    kept_rows = np.unique(np.concatenate([rng.choice(len(new), size=min(n_sample - 8, len(new)), replace=False),
                                          np.arange(len(new) - tail, len(new))]))
    kpos = new[kept_rows]
    kloc = np.array([loc[int(p)] for p in kpos])
    xq = prec.store(O.rmsnorm(h[kloc], w["g_attn"], sh.rms_eps))
    q = prec.store(O.rope_rotate(O.project(xq, w["w_q"]).reshape(-1, hq, dh), kpos, sh.rope_base))
    att = prec.store(O.causal_attention(q, fk, fv, kpos)).reshape(len(kpos), hq * dh)
    assert_close(rec.out_sel[kept_rows], att, "bf16", f"attention output layer {layer + 1}")
    h_next = O.layer_rest(sh, w, prec, h, kloc, rec.out_sel[kept_rows])
    assert_close(rec.hidden_out[kept_rows], h_next, "bf16", f"layer output layer {layer + 1}",
                 scale=ffn_tol_scale(sh.ffn_dim))


def check_chunk_cache(wl, layer, w, h, k_dev, v_dev):
    """A chunk's cache is its own prefill at positions 0..: K/V of every row of the chunk at
    `layer` against the oracle fed with the GPU's input rows h of that layer."""
    sh = wl.shape
    prec = O.Precision("bf16")
    n = h.shape[0]
    x = prec.store(O.rmsnorm(h, w["g_attn"], sh.rms_eps))
    pos = np.arange(n)
    k = prec.store(O.rope_rotate(O.project(x, w["w_k"]).reshape(n, sh.n_kv_heads, sh.head_dim), pos, sh.rope_base))
    v = prec.store(O.project(x, w["w_v"]).reshape(n, sh.n_kv_heads, sh.head_dim))
    assert_close(to_np(k_dev), k, "bf16", f"chunk-0 cache K layer {layer + 1}")
    assert_close(to_np(v_dev), v, "bf16", f"chunk-0 cache V layer {layer + 1}")


def check_decode_teacher_forced(eng, buf, fused, wl, W, emb, tok):
    """One decode step of token `tok` at position N (after a blended prefill of N rows whose
    fused K/V sit in `fused`), run layer by layer; at every layer the attention output, the
    appended K/V row and the layer output of the new row are checked against the oracle's
    decode layer fed the GPU's input row of that layer and the GPU's fused rows."""
    import torch
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import _ptr
    sh = wl.shape
    prec = O.Precision("bf16")
    n = wl.n_tokens
    cs = eng.compute
    with torch.cuda.stream(cs):
        buf.tokens[:1].copy_(torch.tensor([tok], dtype=torch.int32))
        buf.init_sel[:1].copy_(torch.tensor([n], dtype=torch.int32))
    L.cb_embed(eng.ctx, _ptr(buf.tokens), 1, _ptr(eng.emb), _ptr(buf.hidden[0]))
    ws = buf.ws
    cur = 0
    for l in range(sh.n_layers):
        h_in, h_out = buf.hidden[cur], buf.hidden[1 - cur]
        cs.synchronize()
        hin = h_in[:1].cpu().numpy().astype(np.float64)
        fk, fv = to_np(fused[l][0][:n]), to_np(fused[l][1][:n])
        L.cb_decode_layer(eng.ctx, l, _ptr(h_in), _ptr(fused[l][0]), _ptr(fused[l][1]), n, 1, _ptr(buf.init_sel),
                          _ptr(buf.out_sel), _ptr(ws), ws.numel())
        L.cb_layer_rest(eng.ctx, l, _ptr(h_in), 1, _ptr(buf.iota), 1, _ptr(buf.out_sel), _ptr(h_out), _ptr(ws),
                        ws.numel())
        cs.synchronize()
        zero = np.zeros((1,) + fk.shape[1:])
        r = O.blend_layer(sh, W[l], prec, hin, np.concatenate([fk, zero]), np.concatenate([fv, zero]), n,
                          np.array([n]), 1, 0.0)
        out = to_np(buf.out_sel[:1])
        assert_close(out, r["out"].reshape(1, -1), "bf16", f"decode attention output layer {l + 1}")
        assert_close(to_np(fused[l][0][n:n + 1]), r["fused_k"][n:n + 1], "bf16", f"decode K layer {l + 1}")
        assert_close(to_np(fused[l][1][n:n + 1]), r["fused_v"][n:n + 1], "bf16", f"decode V layer {l + 1}")
        ref_h = O.layer_rest(sh, W[l], prec, hin, [0], out)
        assert_close(h_out[:1].cpu().numpy().astype(np.float64), ref_h, "bf16", f"decode layer output {l + 1}",
                     scale=ffn_tol_scale(sh.ffn_dim))
        cur = 1 - cur
