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
