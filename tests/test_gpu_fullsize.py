"""Parity at the benchmark's full size (Qwen2.5-1.5B-shaped, 28 layers, 10 x 512-token chunks +
64 query tokens, 100% -> 30% -> 15%), in the launch configuration bench.py times.

The oracle cannot run the whole prefill in seconds, so at sampled layers it is teacher-forced
with the GPU's own inputs and checks sampled outputs one by one:
  * the deviation of sampled candidate rows (oracle fresh K/V vs the re-rotated GPU cache);
  * the kept set is exactly the top-k of the GPU's deviations (ties to the lower position),
    and the query rows are kept;
  * sampled recomputed rows of the fused cache hold the oracle's fresh K/V; sampled rows that
    were not recomputed hold the re-rotated chunk cache;
  * the attention output and the layer output of sampled kept rows;
and chunk 0's cache at sampled layers is compared with the oracle fed with the GPU's input rows
of that layer (a chunk's cache is its own prefill at positions 0..)."""
import numpy as np
import pytest

import fixtures as F
import oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu

SAMPLED_LAYERS = (0, 1, 2, 27)
N_SAMPLE = 24


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def qwen_run():
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, make_buffers, run_layers
    wl = F.get_config("qwen")
    sh = wl.shape
    eng = Engine(sh, max_tokens=wl.n_tokens + 64)
    for l in range(sh.n_layers):
        eng.load_layer(l, F.layer_weights(sh, l + 1))
    emb = F.embedding(sh)
    eng.load_embedding(emb)
    chunks = F.chunk_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = [(eng.kv_empty(wl.n_tokens), eng.kv_empty(wl.n_tokens)) for _ in range(sh.n_layers)]
    res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                     cache=cache, record=True)
    eng.compute.synchronize()
    hidden_in = [np.asarray(emb[F.all_tokens(wl)], np.float64)] + [r.hidden_out for r in res.records[:-1]]
    return wl, eng, cache, fused, res, hidden_in, chunks, emb


@pytest.mark.parametrize("layer", (0, 1, 27))
def test_chunk_cache_teacher_forced(qwen_run, layer):
    """A chunk's cache is its own prefill at positions 0..: at sampled layers, K/V of every row of
    chunk 0 against the oracle fed with the GPU's input rows of that layer."""
    from rag_kv_cache_amd.pipeline import make_buffers, run_layers
    wl, eng, cache, fused, res, hidden_in, chunks, emb = qwen_run
    sh = wl.shape
    prec = O.Precision("bf16")
    toks = chunks[0]
    n = len(toks)
    buf = make_buffers(eng, n, 0)
    tmp = [(eng.kv_empty(n), eng.kv_empty(n)) for _ in range(sh.n_layers)]
    rec = run_layers(eng, buf, toks, [0], n, [1.0] * sh.n_layers, tmp, record=True).records
    eng.compute.synchronize()
    h = np.asarray(emb[toks], np.float64) if layer == 0 else rec[layer - 1].hidden_out.astype(np.float64)
    w = F.layer_weights(sh, layer + 1)
    x = prec.store(O.rmsnorm(h, w["g_attn"], sh.rms_eps))
    pos = np.arange(n)
    k = prec.store(O.rope_rotate(O.project(x, w["w_k"]).reshape(n, sh.n_kv_heads, sh.head_dim), pos, sh.rope_base))
    v = prec.store(O.project(x, w["w_v"]).reshape(n, sh.n_kv_heads, sh.head_dim))
    assert_close(_np(cache[layer][0][:n]), k, "bf16", f"chunk-0 cache K layer {layer + 1}")
    assert_close(_np(cache[layer][1][:n]), v, "bf16", f"chunk-0 cache V layer {layer + 1}")
    # the bench's cache is the same computation: bit-identical to this re-run
    assert np.array_equal(tmp[layer][0].float().cpu().numpy(), cache[layer][0][:n].float().cpu().numpy())


@pytest.mark.parametrize("layer", SAMPLED_LAYERS)
def test_sampled_layer_teacher_forced(qwen_run, layer):
    wl, eng, cache, fused, res, hidden_in, chunks, emb = qwen_run
    sh = wl.shape
    prec = O.Precision("bf16")
    w = F.layer_weights(sh, layer + 1)
    rec = res.records[layer]
    sel, new = rec.sel, rec.new_sel
    n_ctx, n_q = wl.n_ctx, wl.n_query
    n_cand = len(sel) - n_q
    k = O.k_for_ratio(wl.schedule[layer], n_ctx, n_cand)
    offs = F.chunk_offsets(wl)
    rng = np.random.default_rng(100 + layer)
    hq, hkv, dh = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    h = hidden_in[layer]
    assert h.shape[0] == len(sel)

    # 1. kept set = exact top-k of the GPU deviations (float32, ties to the lower position)
    dev = rec.deviation.astype(np.float32)
    assert len(new) == k + n_q
    assert np.array_equal(new[k:], np.arange(n_ctx, n_ctx + n_q))
    assert np.array_equal(new[:k], np.sort(sel[:n_cand][O.topk_select(dev, k)]))

    # 2. sampled candidate rows: oracle deviation against the re-rotated GPU cache row
    rows = rng.choice(n_cand, size=min(N_SAMPLE, n_cand), replace=False)
    pos = sel[rows]
    chunk_of = np.searchsorted(offs, pos, side="right") - 1
    kc = _np(cache[layer][0])[pos]
    vc = _np(cache[layer][1])[pos]
    k_rot = prec.store(O.rope_rotate(kc, offs[chunk_of], sh.rope_base))
    x = prec.store(O.rmsnorm(h[rows], w["g_attn"], sh.rms_eps))
    k_new = prec.store(O.rope_rotate(O.project(x, w["w_k"]).reshape(-1, hkv, dh), pos, sh.rope_base))
    v_new = prec.store(O.project(x, w["w_v"]).reshape(-1, hkv, dh))
    d_ref = O.kv_deviation(k_new, v_new, k_rot, vc)
    err = np.abs(dev[rows] - d_ref) - 1e-3 * d_ref
    assert err.max() <= 1e-3, f"deviation err {err.max():.3e}"

    # 3. fused cache: recomputed rows hold fresh K/V; other context rows the re-rotated cache
    fk, fv = _np(fused[layer][0]), _np(fused[layer][1])
    assert_close(fk[pos], k_new, "bf16", "fused K of recomputed rows")
    assert_close(fv[pos], v_new, "bf16", "fused V of recomputed rows")
    untouched = np.setdiff1d(np.arange(n_ctx), sel)
    if len(untouched):
        urows = rng.choice(untouched, size=min(N_SAMPLE, len(untouched)), replace=False)
        uchunk = np.searchsorted(offs, urows, side="right") - 1
        rot = prec.store(O.rope_rotate(_np(cache[layer][0])[urows], offs[uchunk], sh.rope_base))
        assert_close(fk[urows], rot, "bf16", "re-rotated K of untouched rows")
        assert np.array_equal(fv[urows], _np(cache[layer][1])[urows])

    # 4. sampled kept rows (always some query rows): attention output and layer output
    loc = {int(p): i for i, p in enumerate(sel)}
    kept_rows = np.unique(np.concatenate([rng.choice(len(new), size=min(N_SAMPLE - 8, len(new)), replace=False),
                                          np.arange(len(new) - 8, len(new))]))
    kpos = new[kept_rows]
    kloc = np.array([loc[int(p)] for p in kpos])
    xq = prec.store(O.rmsnorm(h[kloc], w["g_attn"], sh.rms_eps))
    q = prec.store(O.rope_rotate(O.project(xq, w["w_q"]).reshape(-1, hq, dh), kpos, sh.rope_base))
    att = prec.store(O.causal_attention(q, fk, fv, kpos)).reshape(len(kpos), hq * dh)
    assert_close(rec.out_sel[kept_rows], att, "bf16", f"attention output layer {layer + 1}")
    h_next = O.layer_rest(sh, w, prec, h, kloc, rec.out_sel[kept_rows])
    assert_close(rec.hidden_out[kept_rows], h_next, "bf16", f"layer output layer {layer + 1}")


def test_final_rows_are_the_query_and_kept_rows(qwen_run):
    wl, eng, cache, fused, res, hidden_in, chunks, emb = qwen_run
    sel = res.sel[: res.n_final].cpu().numpy()
    assert res.n_final == 768 + 64
    assert np.all(np.diff(sel) > 0)
    assert np.array_equal(sel[-64:], np.arange(5120, 5184))
    assert np.isfinite(res.hidden[: res.n_final].cpu().numpy()).all()
