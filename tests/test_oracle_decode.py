"""Pins of the oracle's decode step on the fused KV: it must reduce to the textbook forward
when the prefill recomputed everything, and be causal (tokens decoded together or one by one
give the same result)."""
import numpy as np

import fixtures as F
import oracle as O


def _setup():
    wl = F.get_config("tiny3")
    sh = wl.shape
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    return wl, sh, W, F.embedding(sh)


def test_decode_after_full_recompute_is_full_prefill():
    wl, sh, W, E = _setup()
    r = O.blended_prefill(sh, W, E, F.chunk_tokens(wl), F.query_tokens(wl), [1.0] * sh.n_layers)
    fused = [(L["fused_k"], L["fused_v"]) for L in r["layers"]]
    new = np.array([17, 503, 4], dtype=np.int64)
    d = O.decode_step(sh, W, E, O.F64, fused, wl.n_tokens, new)
    full = O.full_prefill(sh, W, E, np.concatenate([F.all_tokens(wl), new]))
    for l in range(sh.n_layers):
        np.testing.assert_allclose(d["fused"][l][0], full["k"][l], atol=1e-12)
        np.testing.assert_allclose(d["fused"][l][1], full["v"][l], atol=1e-12)
    np.testing.assert_allclose(d["hidden"], full["hidden"][-1][-len(new):], atol=1e-12)


def test_decode_is_causal():
    wl, sh, W, E = _setup()
    r = O.blended_prefill(sh, W, E, F.chunk_tokens(wl), F.query_tokens(wl), wl.schedule)
    fused = [(L["fused_k"], L["fused_v"]) for L in r["layers"]]
    n = wl.n_tokens
    both = O.decode_step(sh, W, E, O.F64, fused, n, [11, 22])
    one = O.decode_step(sh, W, E, O.F64, fused, n, [11])
    two = O.decode_step(sh, W, E, O.F64, one["fused"], n + 1, [22])
    np.testing.assert_allclose(both["hidden"][0], one["hidden"][0], atol=1e-12)
    np.testing.assert_allclose(both["hidden"][1], two["hidden"][0], atol=1e-12)
    for l in range(sh.n_layers):
        np.testing.assert_allclose(both["fused"][l][0], two["fused"][l][0], atol=1e-12)
