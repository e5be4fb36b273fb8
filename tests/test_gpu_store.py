"""GPU checks of the chunk-cache producer and store: entries produced through the library
equal the chunk caches (bit for bit: same kernels) and the oracle's chunk caches (tolerance),
a blended prefill fetched from the store equals one fetched from separately pinned caches and
matches the oracle, and an evicted chunk is missed and produced again identically."""
import ctypes

import numpy as np
import pytest
import torch

import fixtures as F
import oracle as O
from parity_util import assert_close, check_selected
from gpu_setup import bits, engine, fused_buffers, weights

pytestmark = pytest.mark.gpu


def _entry(store, slot, layer, eng, n):
    """The stored K and V rows of one entry and layer, as raw bits and as float64."""
    k, v, m = store_layer(store, slot, layer)
    assert m == n
    s = eng.shape
    nb = n * s.n_kv_heads * s.head_dim * (2 if eng.dtype == torch.bfloat16 else 4)
    out = []
    for a in (k, v):
        raw = ctypes.string_at(a, nb)
        if eng.dtype == torch.bfloat16:
            b = np.frombuffer(raw, np.int16).reshape(n, s.n_kv_heads, s.head_dim)
            f = (b.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        else:
            b = np.frombuffer(raw, np.float32).reshape(n, s.n_kv_heads, s.head_dim)
            f = b.astype(np.float64)
        out.append((b.copy(), f))
    return out


def store_layer(store, slot, layer):
    from rag_kv_cache_amd import _lib as L
    return L.cb_store_layer(store.handle, slot, layer)


@pytest.mark.parametrize("cfg", ["tiny", "small_bf16"])
def test_produced_entries_equal_chunk_caches_and_oracle(cfg):
    from rag_kv_cache_amd.pipeline import ChunkStore, build_chunk_caches, produce_chunks
    wl = F.get_config(cfg)
    sh = wl.shape
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    print(f"[store] {cfg}: {len(chunks)} chunks {wl.chunk_lens}", flush=True)
    store = ChunkStore(eng, max(wl.chunk_lens), len(chunks), pinned=True)
    slots = produce_chunks(eng, store, chunks)
    assert sorted(slots) == list(range(len(chunks)))
    cache, _ = build_chunk_caches(eng, chunks)
    offs = F.chunk_offsets(wl)
    W, E = weights(cfg)
    prec = O.Precision.for_dtype(sh.dtype)
    for c, toks in enumerate(chunks):
        ref = O.chunk_caches(sh, W, E, [toks], prec)[0] if c < 2 else None
        for l in range(sh.n_layers):
            (kb, kf), (vb, vf) = _entry(store, slots[c], l, eng, len(toks))
            assert np.array_equal(kb, bits(cache[l][0][offs[c]:offs[c + 1]])), f"chunk {c} layer {l} K"
            assert np.array_equal(vb, bits(cache[l][1][offs[c]:offs[c + 1]])), f"chunk {c} layer {l} V"
            if ref is not None:
                tol = "bf16" if sh.dtype == "bf16" else "f32"
                assert_close(kf, ref[l][0], tol, f"chunk {c} layer {l} K vs oracle")
                assert_close(vf, ref[l][1], tol, f"chunk {c} layer {l} V vs oracle")
    st = store.stats()
    assert (st.entries, st.evictions) == (len(chunks), 0)
    store.close()
    eng.close()


def test_prefill_from_store_equals_pinned_caches_and_oracle():
    from rag_kv_cache_amd.pipeline import ChunkStore, build_chunk_caches, make_buffers, produce_chunks, run_layers
    cfg = "tiny3"
    wl = F.get_config(cfg)
    sh = wl.shape
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    store = ChunkStore(eng, max(wl.chunk_lens), len(chunks) + 2, pinned=True)
    produce_chunks(eng, store, chunks)
    slots = store.lookup_prompt(chunks, hold=True)
    assert slots is not None
    _, host = build_chunk_caches(eng, chunks, pinned_host=True, keep_device=False)
    outs = []
    for hc in (store.host_cache(slots), host):
        buf = make_buffers(eng, wl.n_tokens, len(chunks))
        fused = fused_buffers(eng, wl.n_tokens)
        res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                         host_cache=hc, record=True)
        eng.compute.synchronize()
        outs.append((res, [(bits(k), bits(v)) for k, v in fused]))
    for s in slots:
        store.release(s)
    (r0, f0), (r1, f1) = outs
    assert r0.n_final == r1.n_final
    assert np.array_equal(r0.hidden[: r0.n_final].cpu().numpy(), r1.hidden[: r1.n_final].cpu().numpy())
    for (a, b), (c, d) in zip(f0, f1):
        assert np.array_equal(a, c) and np.array_equal(b, d)
    W, E = weights(cfg)
    ref = O.blended_prefill(sh, W, E, chunks, F.query_tokens(wl), wl.schedule)
    for l, (rec, Lr) in enumerate(zip(r0.records, ref["layers"])):
        n_cand = len(Lr["sel"]) - wl.n_query
        assert np.array_equal(rec.sel, Lr["sel"]), f"layer {l}: S_l differs"
        assert check_selected(rec.new_sel, Lr["new_sel"], Lr["deviation"], Lr["sel"][:n_cand], Lr["k"],
                              wl.n_query) == 0
        assert_close(rec.hidden_out, Lr["hidden_out"], "f32", f"hidden out layer {l}")
    assert np.array_equal(r0.sel[: r0.n_final].cpu().numpy(), ref["sel"])
    store.close()
    eng.close()


def test_eviction_and_reproduction():
    from rag_kv_cache_amd.pipeline import ChunkStore, produce_chunks
    cfg = "tiny"
    wl = F.get_config(cfg)
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    extra = (chunks[0] + 7) % wl.shape.vocab
    store = ChunkStore(eng, max(max(wl.chunk_lens), len(extra)), 2, pinned=True)
    s0 = produce_chunks(eng, store, [chunks[0]])[0]
    first = [(_entry(store, s0, l, eng, len(chunks[0]))) for l in range(wl.shape.n_layers)]
    produce_chunks(eng, store, [chunks[1], extra])   # the store holds 2: chunks[0] is evicted
    assert store.lookup(chunks[0]) == -1
    assert store.lookup(chunks[1]) >= 0 and store.lookup(extra) >= 0
    held = store.lookup(extra, hold=True)            # held: the next insert must evict chunks[1]
    s0b = produce_chunks(eng, store, [chunks[0]])[0]
    assert store.lookup(chunks[1]) == -1 and store.lookup(extra) == held
    for l in range(wl.shape.n_layers):
        again = _entry(store, s0b, l, eng, len(chunks[0]))
        for (a, _), (b, _) in zip(first[l], again):
            assert np.array_equal(a, b)
    st = store.stats()
    assert st.evictions == 2 and st.entries == 2
    store.release(held)
    store.close()
    eng.close()
