"""Pins of the oracle's selection variants from the KVBoost page (section on seam repair):
the cosine deviation of the deviation-guided strategy and the boundary windows of the spatial
strategy.  Each is checked against closed forms, hand-worked examples or a special case the
method reduces to, not against a retyping of its own formula."""
import math

import numpy as np
import pytest

import fixtures as F
import oracle as O


def _rows(a):
    """[n, H_kv, d_h] rows from [n, 2 * H_kv * d_h / 2] data: K half then V half."""
    a = np.asarray(a, np.float64)
    n, w = a.shape
    return a[:, : w // 2].reshape(n, 2, -1), a[:, w // 2:].reshape(n, 2, -1)


def test_cosine_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32))
    k, v = _rows(x)
    assert np.allclose(O.cosine_deviation(k, v, k, v), 0.0, atol=1e-15)            # identical rows
    assert np.allclose(O.cosine_deviation(-k, -v, k, v), 2.0, atol=1e-15)          # opposite rows
    assert np.allclose(O.cosine_deviation(3.5 * k, 3.5 * v, k, v), 0.0, atol=1e-15)  # scale invariance
    # orthogonal rows: disjoint supports
    e1 = np.zeros((1, 32)); e1[0, 3] = 2.0
    e2 = np.zeros((1, 32)); e2[0, 20] = -1.5
    assert np.allclose(O.cosine_deviation(*_rows(e1), *_rows(e2)), 1.0, atol=1e-15)


@pytest.mark.parametrize("theta", [0.1, 0.7, 1.3, 2.9])
def test_cosine_of_a_plane_rotation(theta):
    """Rotating a vector by theta inside a coordinate plane (any pair of coordinates, here one
    in K and one in V) gives deviation 1 - cos(theta), for any norm."""
    a = np.zeros((1, 16)); a[0, 2] = 1.7; a[0, 11] = 0.0
    b = np.zeros((1, 16)); b[0, 2] = 1.7 * math.cos(theta); b[0, 11] = 1.7 * math.sin(theta)
    d = O.cosine_deviation(*_rows(b), *_rows(a))
    assert abs(d[0] - (1.0 - math.cos(theta))) < 1e-14


def test_cosine_zero_rows():
    z = np.zeros((1, 8)); o = np.ones((1, 8))
    assert O.cosine_deviation(*_rows(z), *_rows(z))[0] == 0.0
    assert O.cosine_deviation(*_rows(o), *_rows(z))[0] == 1.0
    assert O.cosine_deviation(*_rows(z), *_rows(o))[0] == 1.0


def test_seam_positions_hand_worked():
    # chunks [0,5) [5,12), 3 query rows, window 2: rows 3,4 | 10,11 | query 12,13,14
    assert O.seam_positions([0, 5, 12], 3, 2).tolist() == [3, 4, 10, 11, 12, 13, 14]
    # a window longer than a chunk covers that chunk only
    assert O.seam_positions([0, 1, 4], 1, 2).tolist() == [0, 2, 3, 4]
    # window 0: only the query rows
    assert O.seam_positions([0, 5, 12], 2, 0).tolist() == [12, 13]
    # no chunk
    assert O.seam_positions([0], 3, 16).tolist() == [0, 1, 2]


def test_seam_prefill_on_a_single_chunk_is_exact():
    """One chunk at offset 0 is an exact prefix: recomputing only its seam window and the query
    at every layer still reproduces full prefill's query rows and the cache."""
    wl = F.get_config("tiny3")
    sh = wl.shape
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    E = F.embedding(sh)
    chunk, q = F.chunk_tokens(wl)[0], F.query_tokens(wl)
    sel = O.seam_positions([0, len(chunk)], len(q), 16)
    r = O.blended_prefill(sh, W, E, [chunk], q, [1.0] * sh.n_layers, initial_sel=sel)
    full = O.full_prefill(sh, W, E, np.concatenate([chunk, q]))
    for l, L in enumerate(r["layers"]):
        assert np.array_equal(L["sel"], sel)                       # the set stays fixed
        np.testing.assert_allclose(L["fused_k"], full["k"][l], atol=1e-12)
        np.testing.assert_allclose(L["fused_v"], full["v"][l], atol=1e-12)
    np.testing.assert_allclose(r["hidden"], full["hidden"][-1][sel], atol=1e-12)


def test_cosine_ranking_matches_brute_force():
    """blend_layer with the cosine score keeps the k rows of largest cosine deviation (ties to
    the lower position), checked by sorting the brute-force cosines on a small prompt with a
    perturbed cache."""
    wl = F.get_config("tiny")
    sh = wl.shape
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    E = F.embedding(sh)
    offs = F.chunk_offsets(wl)
    caches = O.chunk_caches(sh, W, E, F.chunk_tokens(wl))
    fk, fv = O.fuse_cache(sh, O.F64, [c[1] for c in caches], offs, wl.n_query)
    rng = np.random.default_rng(11)
    fk = fk + 0.05 * rng.standard_normal(fk.shape)
    hidden = rng.standard_normal((wl.n_tokens, sh.d_model))
    sel = np.arange(wl.n_tokens)
    r = O.blend_layer(sh, W[1], O.F64, hidden, fk, fv, wl.n_ctx, sel, wl.n_query, 0.3, score="cosine")
    n_cand = wl.n_ctx
    a = np.concatenate([r["k_new"][:n_cand].reshape(n_cand, -1), r["v_new"][:n_cand].reshape(n_cand, -1)], 1)
    b = np.concatenate([fk[:n_cand].reshape(n_cand, -1), fv[:n_cand].reshape(n_cand, -1)], 1)
    cos = [1.0 - float(np.dot(a[i], b[i])) / math.sqrt(float(np.dot(a[i], a[i])) * float(np.dot(b[i], b[i])))
           for i in range(n_cand)]
    k = O.k_for_ratio(0.3, wl.n_ctx, n_cand)
    brute = sorted(range(n_cand), key=lambda i: (-np.float32(cos[i]), i))[:k]
    assert r["new_sel"][:k].tolist() == sorted(brute)
