"""GPU parity of the int8-weight variant (symmetric int8 per output channel, scales applied to the
fp32 sums) against the oracle running the dequantized model (q * s in float32):
  * the bf16 test shape (3 layers, ragged chunks, split-K products with scales in the reduce),
    every layer teacher-forced on the GPU's own inputs, plus a decode step (the int8 skinny
    product);
  * the Yi-34B shape (d_model 7,168, FFN 20,480, GQA group 7) at its real per-layer sizes: the
    first three layers teacher-forced on every row and a decode step layer by layer."""
from dataclasses import replace

import numpy as np
import pytest

import fixtures as F
import oracle as O
from parity_util import assert_close, check_selected, local_index
from gpu_setup import to_np
from layer_checks import check_decode_teacher_forced, check_layer

pytestmark = pytest.mark.gpu


def _engine_i8(sh, max_tokens):
    from rag_kv_cache_amd.pipeline import Engine
    eng = Engine(sh, max_tokens=max_tokens)
    WQ = [F.layer_weights_int8(sh, l) for l in range(1, sh.n_layers + 1)]
    for l in range(sh.n_layers):
        eng.load_layer_int8(l, WQ[l])
    E = F.embedding(sh)
    eng.load_embedding(E)
    return eng, [O.dequantize(w) for w in WQ], E


def test_int8_layers_teacher_forced_and_decode():
    from rag_kv_cache_amd.pipeline import build_chunk_caches, decode, make_buffers, run_layers
    wl = F.get_config("small_bf16")
    sh = wl.shape
    eng, W, E = _engine_i8(sh, wl.n_tokens + 8)
    prec = O.Precision("bf16")
    chunks = F.chunk_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    ref_caches = O.chunk_caches(sh, W, E, chunks, prec)
    for l in range(sh.n_layers):
        assert_close(to_np(cache[l][0]), np.concatenate([c[l][0] for c in ref_caches]), "bf16", f"cache K {l}")
        assert_close(to_np(cache[l][1]), np.concatenate([c[l][1] for c in ref_caches]), "bf16", f"cache V {l}")
    n = wl.n_tokens
    buf = make_buffers(eng, n + 2, len(chunks))
    fused = [(eng.kv_empty(n + 2), eng.kv_empty(n + 2)) for _ in range(sh.n_layers)]
    res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                     cache=cache, record=True)
    eng.compute.synchronize()
    offs = F.chunk_offsets(wl)
    hidden = np.asarray(E[F.all_tokens(wl)], np.float64)
    for l, rec in enumerate(res.records):
        gpu_cache = [(to_np(cache[l][0])[offs[c]:offs[c + 1]], to_np(cache[l][1])[offs[c]:offs[c + 1]])
                     for c in range(len(chunks))]
        fk, fv = O.fuse_cache(sh, prec, gpu_cache, offs, wl.n_query)
        r = O.blend_layer(sh, W[l], prec, hidden, fk, fv, wl.n_ctx, rec.sel, wl.n_query, wl.schedule[l],
                          new_sel_override=rec.new_sel)
        r_own = O.blend_layer(sh, W[l], prec, hidden, fk, fv, wl.n_ctx, rec.sel, wl.n_query, wl.schedule[l])
        n_cand = len(rec.sel) - wl.n_query
        err = np.abs(rec.deviation - r["deviation"]) - 1e-3 * np.abs(r["deviation"])
        assert err.max(initial=0.0) <= 1e-3, f"layer {l}: deviation err {err.max():.2e}"
        check_selected(rec.new_sel, r_own["new_sel"], r_own["deviation"], rec.sel[:n_cand], r_own["k"], wl.n_query)
        assert_close(to_np(fused[l][0])[:n], r["fused_k"], "bf16", f"fused K layer {l}")
        assert_close(to_np(fused[l][1])[:n], r["fused_v"], "bf16", f"fused V layer {l}")
        assert_close(rec.out_sel, r["out"], "bf16", f"attention out layer {l}")
        h_ref = O.layer_rest(sh, W[l], prec, hidden, local_index(rec.sel, rec.new_sel), rec.out_sel)
        assert_close(rec.hidden_out, h_ref, "bf16", f"hidden out layer {l}")
        hidden = rec.hidden_out.astype(np.float64)
    # a decode step of two tokens (the int8 skinny product) against the oracle's decode step
    past = [(to_np(k)[:n], to_np(v)[:n]) for k, v in fused]
    h = decode(eng, buf, [7, 1234], n, fused)
    eng.compute.synchronize()
    got = to_np(h)
    ref = O.decode_step(sh, W, E, prec, past, n, [7, 1234])
    assert_close(got, ref["hidden"], "bf16", "int8 decode hidden")
    eng.close()


def test_int8_yi_shape_teacher_forced():
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    base = F.get_config("yi_r15")
    wl = replace(base, shape=replace(base.shape, n_layers=3), schedule=base.schedule[:3])
    sh = wl.shape
    print(f"[int8] {sh.name}: d {sh.d_model}, ffn {sh.ffn_dim}, {wl.n_tokens} rows", flush=True)
    eng, W, E = _engine_i8(sh, wl.n_tokens + 4)
    chunks = F.chunk_tokens(wl)
    tokens = F.all_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    n = wl.n_tokens
    buf = make_buffers(eng, n + 1, len(chunks))
    fused = [(eng.kv_empty(n + 1), eng.kv_empty(n + 1)) for _ in range(sh.n_layers)]
    res = run_layers(eng, buf, tokens, F.chunk_offsets(wl), wl.n_query, wl.schedule, fused, cache=cache, record=True)
    eng.compute.synchronize()
    hidden_in = [np.asarray(E[tokens], np.float64)] + [r.hidden_out for r in res.records[:-1]]
    for layer in range(sh.n_layers):
        print(f"[int8] layer {layer + 1}: {len(res.records[layer].sel)} -> {len(res.records[layer].new_sel)} rows",
              flush=True)
        check_layer(wl, layer, W[layer], res.records[layer], hidden_in[layer], cache[layer], fused[layer])
    check_decode_teacher_forced(eng, buf, fused, wl, W, E, 11)
    eng.close()
