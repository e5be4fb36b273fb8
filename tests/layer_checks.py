"""Teacher-forced checks of single layers of a large blended prefill against the oracle, on
every row.

At sizes where the oracle cannot run a whole prefill in seconds, each checked layer is fed the
GPU's own inputs of that layer (the residual rows entering it and the chunk cache the GPU
built), and every output of the layer is compared with the oracle's:
  * the deviation of every candidate row: against the oracle's arithmetic on the GPU's own fresh
    rows (1e-3 absolute + 1e-3 relative), and against the oracle's deviation of its own fresh
    rows with a bound of one bf16 rounding step per stored element on either side;
  * the kept set: exactly the top-k of the GPU's deviations (ties to the lower position), and
    the oracle's own top-k of the oracle's deviations except within 1e-3 relative of the k-th
    deviation (the two sides round the fresh K/V independently);
  * every row of the fused cache: the recomputed rows against the oracle's fresh K/V, the others
    against the oracle's re-rotation of the chunk cache (V bit for bit);
  * the attention output of every kept row;
  * the rest of the layer in three pieces, each fed the GPU's own input to that piece: the
    residual after attention h1 = h + out W_o^T, the SwiGLU product of RMSNorm(h1), and the
    layer output h1 + act W_down^T;
and a decode step on the fused KV is checked layer by layer the same way.

Row blocks of the attention run on a thread pool with single-threaded BLAS: each query row's
output depends only on its own query and the keys, so the blocks are the oracle's function on
a subset of rows.  The bf16 bar is the fixed max-abs 2e-2 / rel 1e-2 throughout.
"""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import fixtures as F
import oracle as O
from parity_util import assert_close, check_selected

PREC = O.Precision("bf16")


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _log(msg):
    print(f"[checks] {msg}", flush=True)


def attention_rows(q, fk, fv, pos, block=256):
    """oracle.causal_attention of every row of q (positions pos) over fk, fv, in row blocks."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    n = len(pos)
    out = np.zeros(q.shape)
    starts = list(range(0, n, block))

    def one(s):
        e = min(n, s + block)
        out[s:e] = O.causal_attention(q[s:e], fk, fv, pos[s:e])

    workers = max(1, min(16, os.cpu_count() or 1, len(starts)))
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(one, starts))
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, starts))
    return out


def check_rest(sh, w, what, h, kloc, out_gpu, h1_gpu, act_gpu, h_out_gpu):
    """The rest of a layer in three pieces, each fed the GPU's own input to it."""
    h1_ref = O.attn_residual(w, h, kloc, out_gpu)
    use = {"h1": assert_close(h1_gpu, h1_ref, "bf16", f"{what}: residual after attention")}
    act_ref = O.swiglu(h1_gpu, w, sh.rms_eps, PREC)
    use["swiglu"] = assert_close(act_gpu, act_ref, "bf16", f"{what}: SwiGLU product")
    h_ref = O.mlp(h1_gpu, w, sh.rms_eps, PREC, act=act_gpu)
    use["out"] = assert_close(h_out_gpu, h_ref, "bf16", f"{what}: layer output")
    return use


def check_layer(wl, layer, w, rec, h, cache_kv, fused_kv):
    """wl: the workload; layer: 0-based; w: the oracle's weights of that layer; rec: the GPU's
    LayerRecord (with h1 and act); h: [len(rec.sel), d] residual rows entering the layer (GPU
    values); cache_kv / fused_kv: (K, V) device tensors of the chunk cache and the fused cache."""
    t0 = time.perf_counter()
    sh = wl.shape
    sel, new = np.asarray(rec.sel), np.asarray(rec.new_sel)
    n_ctx, n_q = wl.n_ctx, wl.n_query
    n_cand = len(sel) - n_q
    k = O.k_for_ratio(wl.schedule[layer], n_ctx, n_cand)
    offs = F.chunk_offsets(wl)
    hq, hkv, dh = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    tag = f"{wl.name} layer {layer + 1}"
    assert h.shape[0] == len(sel)

    # the oracle's fresh K/V of every selected row, from the GPU's input rows
    x = PREC.store(O.rmsnorm(h, w["g_attn"], sh.rms_eps))
    k_new = PREC.store(O.rope_rotate(O.project(x, w["w_k"]).reshape(-1, hkv, dh), sel, sh.rope_base))
    v_new = PREC.store(O.project(x, w["w_v"]).reshape(-1, hkv, dh))
    ck, cv = to_np(cache_kv[0]), to_np(cache_kv[1])
    fk, fv = to_np(fused_kv[0]), to_np(fused_kv[1])
    # the oracle's re-rotation of the GPU's chunk cache (every context row)
    ctx_rows = np.arange(n_ctx)
    chunk_of = np.searchsorted(offs, ctx_rows, side="right") - 1
    k_rot = PREC.store(O.rope_rotate(ck, offs[chunk_of], sh.rope_base))

    # 1. deviation of every candidate
    pos = sel[:n_cand]
    dev = rec.deviation.astype(np.float32).astype(np.float64)
    d_own = O.kv_deviation(fk[pos], fv[pos], k_rot[pos], cv[pos])
    err = np.abs(dev - d_own) - 1e-3 * d_own
    assert err.max(initial=0.0) <= 1e-3, f"{tag}: deviation of the GPU's fresh rows, err {err.max():.3e}"
    d_ref = O.kv_deviation(k_new[:n_cand], v_new[:n_cand], k_rot[pos], cv[pos])
    # each stored bf16 element of either side may sit one rounding step (at most 2^-7 |x|) away
    # from the other side's, so per element the squared difference moves by at most e (2 |delta| + e)
    slack = np.zeros(n_cand)
    for a, b in ((k_new[:n_cand], k_rot[pos]), (v_new[:n_cand], cv[pos])):
        e = 2.0 ** -7 * (np.abs(a) + np.abs(b))
        slack += (e * (2 * np.abs(a - b) + e)).sum(axis=(1, 2))
    err = np.abs(dev - d_ref) - 1e-3 * d_ref - slack
    assert err.max(initial=0.0) <= 1e-3, f"{tag}: deviation err {err.max():.3e} beyond the rounding bound"

    # 2. kept set: the top-k of the GPU's own deviations, and the oracle's top-k up to the tie band
    assert len(new) == k + n_q
    assert np.array_equal(new[k:], np.arange(n_ctx, n_ctx + n_q)), f"{tag}: query rows"
    assert np.array_equal(new[:k], np.sort(pos[O.topk_select(rec.deviation.astype(np.float32), k)])), \
        f"{tag}: kept set is not the top-k of the GPU's deviations"
    ref_new = np.concatenate([np.sort(pos[O.topk_select(d_ref, k)]), np.arange(n_ctx, n_ctx + n_q)])
    flips = check_selected(new, ref_new, d_ref, pos, k, n_q)

    # 3. every row of the fused cache
    assert_close(fk[sel], k_new, "bf16", f"{tag}: fused K of recomputed rows")
    assert_close(fv[sel], v_new, "bf16", f"{tag}: fused V of recomputed rows")
    untouched = np.setdiff1d(ctx_rows, sel)
    if len(untouched):
        assert_close(fk[untouched], k_rot[untouched], "bf16", f"{tag}: re-rotated K of rows not recomputed")
        assert np.array_equal(fv[untouched], cv[untouched]), f"{tag}: V of rows not recomputed"

    # 4. Q of every kept row against the oracle's Q of the GPU's input rows; the attention output
    #    of every kept row against the oracle's attention of the GPU's Q over the GPU's fused rows
    loc = {int(p): i for i, p in enumerate(sel)}
    kloc = np.array([loc[int(p)] for p in new], dtype=np.int64)
    q = PREC.store(O.rope_rotate(O.project(x[kloc], w["w_q"]).reshape(-1, hq, dh), new, sh.rope_base))
    use = {"q": assert_close(rec.q, q.reshape(len(new), hq * dh), "bf16", f"{tag}: Q of the kept rows")}
    att = PREC.store(attention_rows(rec.q.astype(np.float64).reshape(-1, hq, dh), fk, fv, new))
    att = att.reshape(len(new), hq * dh)
    use["attention"] = assert_close(rec.out_sel, att, "bf16", f"{tag}: attention output")
    use["attention_max_abs"] = float(np.abs(rec.out_sel - att).max(initial=0.0))

    # 5. rest of the layer, piece by piece
    use.update(check_rest(sh, w, tag, h, kloc, rec.out_sel, rec.h1, rec.act, rec.hidden_out))
    _log(f"{tag}: {len(sel)} -> {len(new)} rows, {flips} tie-band flips, all rows checked "
         f"in {time.perf_counter() - t0:.1f} s; share of the bar used: "
         + ", ".join(f"{k} {v:.3g}" for k, v in use.items()))
    return flips


def check_chunk_cache(wl, layer, w, h, k_dev, v_dev):
    """A chunk's cache is its own prefill at positions 0..: K/V of every row of the chunk at
    `layer` against the oracle fed with the GPU's input rows h of that layer."""
    sh = wl.shape
    n = h.shape[0]
    x = PREC.store(O.rmsnorm(h, w["g_attn"], sh.rms_eps))
    pos = np.arange(n)
    k = PREC.store(O.rope_rotate(O.project(x, w["w_k"]).reshape(n, sh.n_kv_heads, sh.head_dim), pos, sh.rope_base))
    v = PREC.store(O.project(x, w["w_v"]).reshape(n, sh.n_kv_heads, sh.head_dim))
    assert_close(to_np(k_dev), k, "bf16", f"chunk-0 cache K layer {layer + 1}")
    assert_close(to_np(v_dev), v, "bf16", f"chunk-0 cache V layer {layer + 1}")


def check_decode_teacher_forced(eng, buf, fused, wl, W, emb, tok):
    """One decode step of token `tok` at position N (after a blended prefill of N rows whose
    fused K/V sit in `fused`), run layer by layer; at every layer whose weights W holds (a list
    of every layer's, or a dict layer -> weights) the attention output, the appended K/V row and
    the rest of the layer of the new row are checked against the oracle's decode layer fed the
    GPU's input row of that layer and the GPU's fused rows."""
    import torch
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import _ptr, workspace_intermediates, workspace_q
    sh = wl.shape
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
        cs.synchronize()
        q_gpu = workspace_q(eng, ws, 1, 1).astype(np.float64)
        L.cb_layer_rest(eng.ctx, l, _ptr(h_in), 1, _ptr(buf.iota), 1, _ptr(buf.out_sel), _ptr(h_out), _ptr(ws),
                        ws.numel())
        cs.synchronize()
        if isinstance(W, dict) and l not in W:
            cur = 1 - cur
            continue
        h1, act = workspace_intermediates(eng, ws, 1, 1)
        zero = np.zeros((1,) + fk.shape[1:])
        r = O.blend_layer(sh, W[l], PREC, hin, np.concatenate([fk, zero]), np.concatenate([fv, zero]), n,
                          np.array([n]), 1, 0.0)
        out = to_np(buf.out_sel[:1])
        assert_close(q_gpu, r["q"].reshape(1, -1), "bf16", f"decode Q layer {l + 1}")
        fk1 = np.concatenate([fk, to_np(fused[l][0][n:n + 1])])
        fv1 = np.concatenate([fv, to_np(fused[l][1][n:n + 1])])
        att = PREC.store(O.causal_attention(q_gpu.reshape(1, sh.n_q_heads, sh.head_dim), fk1, fv1, [n]))
        assert_close(out, att.reshape(1, -1), "bf16", f"decode attention output layer {l + 1}")
        assert_close(to_np(fused[l][0][n:n + 1]), r["fused_k"][n:n + 1], "bf16", f"decode K layer {l + 1}")
        assert_close(to_np(fused[l][1][n:n + 1]), r["fused_v"][n:n + 1], "bf16", f"decode V layer {l + 1}")
        check_rest(sh, W[l], f"decode layer {l + 1}", hin, [0], out, h1.astype(np.float64),
                   act.astype(np.float64), h_out[:1].cpu().numpy().astype(np.float64))
        cur = 1 - cur
