"""Pins of the oracle's RoPE and position-update arithmetic against closed forms.

CacheBlend explainer, "Position encoding update": a cached K is moved to its new
position by the rotation K_new = R(dp) K_cached.  These tests pin R itself:
rotation algebra, the complex-multiplication form, orthogonality, and the
layer-1 identity that follows from it."""
import numpy as np
import pytest

import fixtures as F
import oracle as O


def _rand(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rotation_composes_additively():
    x = _rand((7, 3, 64))
    a = np.array([0, 1, 5, 17, 300, 4095, 16383])
    b = np.array([3, 0, 11, 2, 1000, 1, 256])
    lhs = O.rope_rotate(O.rope_rotate(x, a, 10000.0), b, 10000.0)
    rhs = O.rope_rotate(x, a + b, 10000.0)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-11)


def test_rotation_identity_and_inverse():
    x = _rand((5, 2, 128), 1)
    np.testing.assert_array_equal(O.rope_rotate(x, np.zeros(5, int), 10000.0), x)
    p = np.array([1, 9, 77, 512, 5000])
    back = O.rope_rotate(O.rope_rotate(x, p, 10000.0), -p, 10000.0)
    np.testing.assert_allclose(back, x, atol=1e-12)


def test_rotation_is_complex_multiplication_half_split():
    # (a_i, b_i) = (x_i, x_{i+d/2}) rotated by angle p*base^(-2i/d) == (a + i b) * e^{i angle}
    dh, base = 64, 10000.0
    x = _rand((4, 1, dh), 2)
    p = np.array([0, 3, 100, 2047])
    y = O.rope_rotate(x, p, base)
    theta = base ** (-np.arange(dh // 2) * 2.0 / dh)
    z = (x[:, 0, : dh // 2] + 1j * x[:, 0, dh // 2:]) * np.exp(1j * p[:, None] * theta[None, :])
    np.testing.assert_allclose(y[:, 0, : dh // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, 0, dh // 2:], z.imag, atol=1e-12)


def test_rotation_known_values():
    # i = 0 has theta = 1: a unit vector on the first pair turns by exactly p radians
    x = np.zeros((1, 1, 8))
    x[0, 0, 0] = 1.0
    y = O.rope_rotate(x, np.array([2]), 10000.0)
    assert y[0, 0, 0] == pytest.approx(np.cos(2.0), abs=1e-15)
    assert y[0, 0, 4] == pytest.approx(np.sin(2.0), abs=1e-15)
    # the last pair i = d/2-1 has theta = base^(-(d-2)/d)
    x = np.zeros((1, 1, 8))
    x[0, 0, 3] = 1.0
    y = O.rope_rotate(x, np.array([1000]), 10000.0)
    ang = 1000 * 10000.0 ** (-6 / 8)
    assert y[0, 0, 3] == pytest.approx(np.cos(ang), abs=1e-13)
    assert y[0, 0, 7] == pytest.approx(np.sin(ang), abs=1e-13)


def test_rotation_preserves_distances():
    # ||R x - R y|| = ||x - y||: deviation is the same before or after RoPE
    x, y = _rand((6, 2, 128), 3), _rand((6, 2, 128), 4)
    p = np.array([0, 1, 2, 600, 5000, 16000])
    dr = O.rope_rotate(x, p, 1e4) - O.rope_rotate(y, p, 1e4)
    np.testing.assert_allclose((dr ** 2).sum((1, 2)), ((x - y) ** 2).sum((1, 2)), rtol=1e-12)


def test_rope_delta_uses_chunk_offset():
    offs = np.array([0, 3, 7, 8])
    k = _rand((8, 2, 16), 5)
    got = O.rope_delta(k, offs, 10000.0)
    want = np.concatenate([O.rope_rotate(k[0:3], [0] * 3, 1e4), O.rope_rotate(k[3:7], [3] * 4, 1e4),
                           O.rope_rotate(k[7:8], [7], 1e4)])
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(got[:3], k[:3])  # chunk 0 sits at offset 0: unchanged


@pytest.mark.parametrize("cfg", ["tiny", "tiny_gqa"])
def test_layer1_identity(cfg):
    """At decoder layer 1 a token's K and V depend only on its embedding and position, so the
    re-rotated chunk cache equals K computed at the shifted position, and V is unchanged."""
    wl = F.get_config(cfg)
    sh = wl.shape
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    E = F.embedding(sh)
    caches = O.chunk_caches(sh, W[:1], E, F.chunk_tokens(wl))
    full = O.full_prefill(sh, W[:1], E, F.all_tokens(wl))
    offs = F.chunk_offsets(wl)
    fk, fv = O.fuse_cache(sh, O.F64, [c[0] for c in caches], offs, wl.n_query)
    n_ctx = wl.n_ctx
    np.testing.assert_allclose(fk[:n_ctx], full["k"][0][:n_ctx], atol=1e-12)
    np.testing.assert_allclose(fv[:n_ctx], full["v"][0][:n_ctx], atol=1e-13)
    # and the cache of a non-first chunk really differs before re-rotation
    raw = np.concatenate([c[0][0] for c in caches])
    assert np.abs(raw[offs[1]:] - full["k"][0][offs[1]:n_ctx]).max() > 1e-2
