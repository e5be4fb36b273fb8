"""GPU parity of decoding with the fused KV (cb_decode_layer) against the oracle: after a
full-recompute prefill it must equal full prefill of the longer prompt; after a blended
prefill it must equal the oracle's decode step fed the GPU's own fused KV."""
import numpy as np
import pytest

import fixtures as F
import oracle as O
from parity_util import assert_close
from gpu_setup import engine, fused_buffers, to_np, weights

pytestmark = pytest.mark.gpu


def _prefill(cfg, schedule, extra):
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    wl = F.get_config(cfg)
    eng = engine(cfg, max_tokens=wl.n_tokens + extra + 8)
    cache, _ = build_chunk_caches(eng, F.chunk_tokens(wl))
    buf = make_buffers(eng, wl.n_tokens + extra, len(wl.chunk_lens))
    fused = fused_buffers(eng, wl.n_tokens + extra)
    run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, schedule, fused, cache=cache)
    eng.compute.synchronize()
    return wl, eng, buf, fused


def test_decode_after_full_recompute_is_full_prefill():
    from rag_kv_cache_amd.pipeline import decode
    cfg = "tiny3"
    wl = F.get_config(cfg)
    new = [[17, 503, 4], [88]]
    wl, eng, buf, fused = _prefill(cfg, [1.0] * wl.shape.n_layers, 4)
    n = wl.n_tokens
    outs = []
    for toks in new:
        h = decode(eng, buf, toks, n, fused)
        eng.compute.synchronize()  # the step runs on the engine's compute stream
        outs.append(to_np(h))
        n += len(toks)
    W, E = weights(cfg)
    full = O.full_prefill(wl.shape, W, E, np.concatenate([F.all_tokens(wl)] + [np.asarray(t) for t in new]))
    assert_close(outs[0], full["hidden"][-1][wl.n_tokens:wl.n_tokens + 3], "f32", "decode step 1 hidden")
    assert_close(outs[1], full["hidden"][-1][wl.n_tokens + 3:], "f32", "decode step 2 hidden")
    for l in range(wl.shape.n_layers):
        assert_close(to_np(fused[l][0])[:n], full["k"][l], "f32", f"fused K layer {l}")
        assert_close(to_np(fused[l][1])[:n], full["v"][l], "f32", f"fused V layer {l}")


@pytest.mark.parametrize("cfg", ["tiny_gqa", "small_bf16"])
def test_decode_on_blended_kv_matches_oracle(cfg):
    from rag_kv_cache_amd.pipeline import decode
    wl = F.get_config(cfg)
    wl, eng, buf, fused = _prefill(cfg, wl.schedule, 3)
    n = wl.n_tokens
    past = [(to_np(k)[:n], to_np(v)[:n]) for k, v in fused]
    toks = [5, 901]
    h = decode(eng, buf, toks, n, fused)
    eng.compute.synchronize()  # the step runs on the engine's compute stream
    got = to_np(h)
    W, E = weights(cfg)
    prec = O.F64 if wl.shape.dtype == "f32" else O.Precision("bf16")
    ref = O.decode_step(wl.shape, W, E, prec, past, n, toks)
    dt = "f32" if wl.shape.dtype == "f32" else "bf16"
    assert_close(got, ref["hidden"], dt, "decode hidden")
    for l in range(wl.shape.n_layers):
        assert_close(to_np(fused[l][0])[n:n + 2], ref["fused"][l][0][n:], dt, f"appended K layer {l}")
        assert_close(to_np(fused[l][1])[n:n + 2], ref["fused"][l][1][n:], dt, f"appended V layer {l}")
        # rows of the prefill are left as they were
        assert np.array_equal(to_np(fused[l][0])[:n], past[l][0])


@pytest.mark.parametrize("group", (1, 2, 4, 6, 7, 8))
@pytest.mark.parametrize("n_new", (1, 2, 3))
def test_decode_every_group_and_row_count(group, n_new):
    """Decode steps of 1, 2 and 3 new rows for every GQA group size the kernels are built for,
    after a 2-layer blended prefill of ragged chunks (632 fused rows: the 128-key ranges of a
    decode step give 5 splits), against the oracle's decode step fed the GPU's fused KV.  The
    few-row vector-ALU kernel takes rows x group <= 8 (rows counted as 1, 2 or 4); the other
    cases run the 16-row MFMA kernel."""
    from dataclasses import replace
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, decode, make_buffers, run_layers
    base = F.get_config("small_bf16")
    sh = replace(base.shape, name=f"small-bf16-g{group}", n_layers=2, n_q_heads=2 * group, n_kv_heads=2)
    wl = F.Workload(f"dec_g{group}", sh, base.chunk_lens, base.n_query, (1.0, 0.30))
    print(f"[decode] group {group}, {n_new} new rows", flush=True)
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    E = F.embedding(sh)
    eng = Engine(sh, max_tokens=wl.n_tokens + 8)
    eng.load_all(lambda l: W[l - 1], E)
    cache, _ = build_chunk_caches(eng, F.chunk_tokens(wl))
    n = wl.n_tokens
    buf = make_buffers(eng, n + 4, len(wl.chunk_lens))
    fused = [(eng.kv_empty(n + 4), eng.kv_empty(n + 4)) for _ in range(sh.n_layers)]
    run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused, cache=cache)
    eng.compute.synchronize()
    past = [(to_np(k)[:n], to_np(v)[:n]) for k, v in fused]
    toks = [17, 1999, 3][:n_new]
    h = decode(eng, buf, toks, n, fused)
    eng.compute.synchronize()  # the step runs on the engine's compute stream
    got = to_np(h)
    ref = O.decode_step(sh, W, E, O.Precision("bf16"), past, n, toks)
    assert_close(got, ref["hidden"], "bf16", f"group {group}: decode hidden")
    for l in range(sh.n_layers):
        assert_close(to_np(fused[l][0])[n:n + n_new], ref["fused"][l][0][n:], "bf16", f"appended K layer {l}")
        assert_close(to_np(fused[l][1])[n:n + n_new], ref["fused"][l][1][n:], "bf16", f"appended V layer {l}")
    eng.close()
