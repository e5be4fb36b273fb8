"""Parity at the larger model shapes' real per-layer sizes: Mistral-7B (4,096 context rows in 6
chunks of 640 + 256 query rows, GQA group 4; recompute ratios 10%, 15% and 20%), Yi-34B (8 x 480
+ 256, group 7, d_model 7,168) and Llama-70B (group 8, d_model 8,192, FFN 28,672) at 4K and at
16K context (32 x 512 + 256 rows: the largest prompt, 16,640 rows through layer 1).

Mistral-7B runs at its full depth of 32 layers (the gradual filter then runs through every
layer) and layers 1, 2, 3, 16 and 32 are checked.  Yi-34B and Llama-70B run their first three
decoder layers (layer 1 at ratio 1, layer 2 narrowing to the ratio, layer 3 at the steady ratio)
with the weights those layers have in the full model: every kernel sees the same sizes at any
depth, so these layers cover the whole model's launch shapes.  The Llama-70B cases, whose cached
KV streams from pinned host memory, also run the prefetched path and must give the same bits.

Each checked layer is compared with the oracle on every row, fed the GPU's own inputs of that
layer (layer_checks.check_layer); then one decode step on the fused KV, each layer against the
oracle's decode layer fed the GPU's input row and fused rows of that layer."""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import replace

import numpy as np
import pytest
import torch

import fixtures as F
from layer_checks import check_chunk_cache, check_decode_teacher_forced, check_layer

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1200)]

CASES = ("mistral_r10", "mistral_r15", "mistral_r20", "yi_r15", "l70_4k", "l70_16k")
FULL_DEPTH = {"mistral-7b": (0, 1, 2, 15, 31)}   # checked layers of the shapes run at full depth
REDUCED_LAYERS = 3

_state = {"shape": None}


def _workload(name):
    """The case's workload: full depth for the shapes in FULL_DEPTH, else its first layers."""
    wl = F.get_config(name)
    if wl.shape.name in FULL_DEPTH:
        return wl
    return replace(wl, shape=replace(wl.shape, n_layers=REDUCED_LAYERS), schedule=wl.schedule[:REDUCED_LAYERS])


def _checked(wl):
    return FULL_DEPTH.get(wl.shape.name, tuple(range(wl.shape.n_layers)))


def _engine(wl):
    """One engine per model shape, kept while its cases run.  The oracle keeps the weights of
    the checked layers only; the draws of three layers run at a time."""
    from rag_kv_cache_amd.pipeline import Engine
    sh = wl.shape
    if _state["shape"] != sh.name:
        if _state.get("eng") is not None:
            _state["eng"].close()
        _state.clear()
        _state["shape"] = None
        max_tok = max(_workload(c).n_tokens for c in CASES if F.get_config(c).shape.name == sh.name) + 2
        print(f"[shapes] loading {sh.name}: d {sh.d_model}, heads {sh.n_q_heads}/{sh.n_kv_heads}, "
              f"ffn {sh.ffn_dim}, {sh.n_layers} layers, up to {max_tok} rows", flush=True)
        eng = Engine(sh, max_tokens=max_tok)
        keep = set(_checked(wl))
        W = {}
        with ThreadPoolExecutor(max_workers=3) as ex:
            for l, w in enumerate(ex.map(lambda i: F.layer_weights(sh, i + 1), range(sh.n_layers))):
                eng.load_layer(l, w)
                if l in keep:
                    W[l] = w
        emb = F.embedding(sh)
        eng.load_embedding(emb)
        torch.cuda.synchronize()
        _state.update(shape=sh.name, eng=eng, W=W, emb=emb)
    return _state["eng"], _state["W"], _state["emb"]


@pytest.fixture(scope="module", autouse=True)
def _release():
    yield
    if _state.get("eng") is not None:
        _state["eng"].close()
    _state.clear()


@pytest.mark.parametrize("name", CASES)
def test_shape_teacher_forced(name):
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    wl = _workload(name)
    sh = wl.shape
    eng, W, emb = _engine(wl)
    print(f"[shapes] {name}: {sh.n_layers} layers, {wl.n_ctx} context + {wl.n_query} query rows, "
          f"checked layers {[l + 1 for l in _checked(wl)]}", flush=True)
    chunks = F.chunk_tokens(wl)
    tokens = F.all_tokens(wl)
    streamed = name.startswith("l70")  # these shapes stream the cached KV from pinned host memory
    cache, host = build_chunk_caches(eng, chunks, pinned_host=streamed)
    buf = make_buffers(eng, wl.n_tokens + 1, len(chunks))
    fused = [(eng.kv_empty(wl.n_tokens + 1), eng.kv_empty(wl.n_tokens + 1)) for _ in range(sh.n_layers)]
    res = run_layers(eng, buf, tokens, F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                     cache=cache, record=True)
    eng.compute.synchronize()
    k = int(np.floor(float(np.float32(wl.schedule[-1])) * wl.n_ctx + 0.5))
    assert res.n_final == k + wl.n_query
    hidden_in = [np.asarray(emb[tokens], np.float64)] + [r.hidden_out for r in res.records[:-1]]
    for layer in _checked(wl):
        print(f"[shapes] {name}: layer {layer + 1}, {len(res.records[layer].sel)} -> "
              f"{len(res.records[layer].new_sel)} rows", flush=True)
        check_layer(wl, layer, W[layer], res.records[layer], hidden_in[layer], cache[layer], fused[layer])
    del hidden_in

    if streamed:  # the pinned-host prefetch path gives the same bits as the HBM-resident one
        buf2 = make_buffers(eng, wl.n_tokens + 1, len(chunks))
        fused2 = [(eng.kv_empty(wl.n_tokens + 1), eng.kv_empty(wl.n_tokens + 1)) for _ in range(sh.n_layers)]
        res2 = run_layers(eng, buf2, tokens, F.chunk_offsets(wl), wl.n_query, wl.schedule, fused2, host_cache=host)
        eng.compute.synchronize()
        assert res2.n_final == res.n_final
        assert np.array_equal(res2.hidden[: res2.n_final].cpu().numpy(), res.hidden[: res.n_final].cpu().numpy())
        for (a, b), (c, d) in zip(fused, fused2):
            assert np.array_equal(a.view(torch.int16).cpu().numpy(), c.view(torch.int16).cpu().numpy())
            assert np.array_equal(b.view(torch.int16).cpu().numpy(), d.view(torch.int16).cpu().numpy())
        del buf2, fused2, host

    # one decode step on the fused KV, layer by layer (the few-row attention over every fused row)
    check_decode_teacher_forced(eng, buf, fused, wl, W, emb, 11)

    if sh.name not in FULL_DEPTH:
        # chunk 0's cache at the last layer: its own prefill at positions 0..
        toks = chunks[0]
        n = len(toks)
        cbuf = make_buffers(eng, n, 0)
        tmp = [(eng.kv_empty(n), eng.kv_empty(n)) for _ in range(sh.n_layers)]
        rec = run_layers(eng, cbuf, toks, [0], n, [1.0] * sh.n_layers, tmp, record=True).records
        eng.compute.synchronize()
        last = sh.n_layers - 1
        check_chunk_cache(wl, last, W[last], rec[last - 1].hidden_out.astype(np.float64),
                          cache[last][0][:n], cache[last][1][:n])
    del cache, fused, buf
