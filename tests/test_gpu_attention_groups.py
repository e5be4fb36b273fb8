"""The bf16 attention for every GQA group size the kernel is instantiated for (1, 2, 4, 6, 7
and 8 query heads per KV head), teacher-forced against the oracle: a 2-layer blended prefill of
ragged chunks (layer 2 keeps 30% of the context); at both layers the attention output of every
kept row equals the oracle's causal attention over the GPU's own fused K/V, with Q computed by
the oracle from the GPU's input rows of that layer."""
from dataclasses import replace

import numpy as np
import pytest

import fixtures as F
import oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu

GROUPS = (1, 2, 4, 6, 7, 8)


def _workload(group):
    sh = replace(F.get_config("small_bf16").shape, name=f"small-bf16-g{group}", n_layers=2, n_q_heads=2 * group, n_kv_heads=2)
    return F.Workload(f"attn_g{group}", sh, (200, 256, 131), 45, (1.0, 0.30))


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("group", GROUPS)
def test_attention_every_group_size(group):
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, make_buffers, run_layers
    wl = _workload(group)
    sh = wl.shape
    print(f"[attn] group {group}: {sh.n_q_heads}/{sh.n_kv_heads} heads, {wl.n_tokens} rows", flush=True)
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    emb = F.embedding(sh)
    eng = Engine(sh, max_tokens=wl.n_tokens + 8)
    eng.load_all(lambda l: W[l - 1], emb)
    chunks = F.chunk_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = [(eng.kv_empty(wl.n_tokens), eng.kv_empty(wl.n_tokens)) for _ in range(sh.n_layers)]
    res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                     cache=cache, record=True)
    eng.compute.synchronize()
    prec = O.Precision("bf16")
    hq, hkv, dh = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    hidden_in = [np.asarray(emb[F.all_tokens(wl)], np.float64), res.records[0].hidden_out]
    for layer, rec in enumerate(res.records):
        w = W[layer]
        loc = {int(p): i for i, p in enumerate(rec.sel)}
        kpos = rec.new_sel
        kloc = np.array([loc[int(p)] for p in kpos])
        x = prec.store(O.rmsnorm(hidden_in[layer][kloc], w["g_attn"], sh.rms_eps))
        q = prec.store(O.rope_rotate(O.project(x, w["w_q"]).reshape(-1, hq, dh), kpos, sh.rope_base))
        att = prec.store(O.causal_attention(q, _np(fused[layer][0]), _np(fused[layer][1]), kpos))
        assert_close(rec.out_sel, att.reshape(len(kpos), hq * dh), "bf16",
                     f"group {group} layer {layer + 1} attention ({len(kpos)} kept rows)")
    eng.close()


@pytest.mark.parametrize("chunk_lens", [(483,) * 6, (503,) * 18], ids=["12_ranges", "36_ranges"])
def test_query_rows_over_a_long_context(chunk_lens):
    """A layer that keeps only the 45 query rows (ratio 0) over a long context: kept sets of at
    most 64 rows get 256-key ranges, so 2,943 rows give 12 ranges and 9,099 rows 36, more than
    the combine's one-round path takes (8): it merges them in batches.  The attention
    output of every query row equals the oracle's causal attention over the GPU's fused K/V,
    with Q from the GPU's input rows of that layer."""
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, make_buffers, run_layers
    sh = replace(F.get_config("small_bf16").shape, name="small-bf16-long", n_layers=2)
    wl = F.Workload(f"long_{len(chunk_lens)}", sh, chunk_lens, 45, (1.0, 0.0))
    print(f"[attn] {wl.n_ctx} context + {wl.n_query} query rows", flush=True)
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    emb = F.embedding(sh)
    eng = Engine(sh, max_tokens=wl.n_tokens + 8)
    eng.load_all(lambda l: W[l - 1], emb)
    chunks = F.chunk_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = [(eng.kv_empty(wl.n_tokens), eng.kv_empty(wl.n_tokens)) for _ in range(sh.n_layers)]
    res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                     cache=cache, record=True)
    eng.compute.synchronize()
    prec = O.Precision("bf16")
    hq, dh = sh.n_q_heads, sh.head_dim
    rec = res.records[1]
    assert rec.new_sel.tolist() == list(range(wl.n_ctx, wl.n_tokens))
    loc = {int(p): i for i, p in enumerate(rec.sel)}
    kpos = rec.new_sel
    kloc = np.array([loc[int(p)] for p in kpos])
    x = prec.store(O.rmsnorm(res.records[0].hidden_out[kloc], W[1]["g_attn"], sh.rms_eps))
    q = prec.store(O.rope_rotate(O.project(x, W[1]["w_q"]).reshape(-1, hq, dh), kpos, sh.rope_base))
    att = prec.store(O.causal_attention(q, _np(fused[1][0]), _np(fused[1][1]), kpos))
    assert_close(rec.out_sel, att.reshape(len(kpos), hq * dh), "bf16", "query-row attention over the long context")
    eng.close()
