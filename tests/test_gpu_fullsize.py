"""Parity at the benchmark's full size (Qwen2.5-1.5B-shaped, 28 layers, 10 x 512-token chunks +
64 query tokens, 100% -> 30% -> 15%), in the launch configuration bench.py times.

The oracle cannot run the whole prefill in seconds, so at layers 1, 2, 3, 14 and 28 it is
teacher-forced with the GPU's own inputs of the layer and every output row is compared
(layer_checks.check_layer): the deviation of every candidate, the kept set against the oracle's
own top-k (tie band 1e-3 of the k-th deviation), every row of the fused cache, the attention
output of every kept row, and the rest of the layer piece by piece.  Chunk 0's cache at layers
1, 2 and 28 is compared with the oracle fed with the GPU's input rows of that layer (a chunk's
cache is its own prefill at positions 0..)."""
import numpy as np
import pytest

import fixtures as F
from layer_checks import check_chunk_cache, check_layer

pytestmark = pytest.mark.gpu

CHECKED_LAYERS = (0, 1, 2, 13, 27)


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
    toks = chunks[0]
    n = len(toks)
    buf = make_buffers(eng, n, 0)
    tmp = [(eng.kv_empty(n), eng.kv_empty(n)) for _ in range(sh.n_layers)]
    rec = run_layers(eng, buf, toks, [0], n, [1.0] * sh.n_layers, tmp, record=True).records
    eng.compute.synchronize()
    h = np.asarray(emb[toks], np.float64) if layer == 0 else rec[layer - 1].hidden_out.astype(np.float64)
    check_chunk_cache(wl, layer, F.layer_weights(sh, layer + 1), h, cache[layer][0][:n], cache[layer][1][:n])
    # the bench's cache is the same computation: bit-identical to this re-run
    assert np.array_equal(tmp[layer][0].float().cpu().numpy(), cache[layer][0][:n].float().cpu().numpy())


@pytest.mark.parametrize("layer", CHECKED_LAYERS)
def test_layer_teacher_forced(qwen_run, layer):
    wl, eng, cache, fused, res, hidden_in, chunks, emb = qwen_run
    check_layer(wl, layer, F.layer_weights(wl.shape, layer + 1), res.records[layer], hidden_in[layer],
                cache[layer], fused[layer])


def test_final_rows_are_the_query_and_kept_rows(qwen_run):
    wl, eng, cache, fused, res, hidden_in, chunks, emb = qwen_run
    sel = res.sel[: res.n_final].cpu().numpy()
    assert res.n_final == 768 + 64
    assert np.all(np.diff(sel) > 0)
    assert np.array_equal(sel[-64:], np.arange(5120, 5184))
    assert np.isfinite(res.hidden[: res.n_final].cpu().numpy()).all()
