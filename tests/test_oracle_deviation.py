"""Pins of the oracle's KV deviation (CacheBlend explainer, "HKVD token selection": the
deviation of a token is the L2 norm of the difference between its cached and its recomputed KV,
over the layer's whole KV) and of the oracle's bfloat16 rounding.

The deviation is checked against values worked out by hand: rows that differ only in V, only in
K, only in the second KV head, in both K and V, and a Pythagorean pair, so that a score that
drops K, V or a head, or takes the norm instead of its square, fails here.  A brute-force
element loop then checks the deviation that blend_layer reports against its own fresh rows and
the fused rows it was given (the re-rotated cache before the scatter), on a tiny layer."""
import numpy as np
import pytest

import fixtures as F
import oracle as O


def _rows(n=1, hkv=2, dh=4):
    return np.zeros((n, hkv, dh)), np.zeros((n, hkv, dh))


def test_deviation_of_rows_differing_only_in_v():
    k0, v0 = _rows()
    k1, v1 = k0.copy(), v0.copy()
    v1[0, 0, :] = [1.0, 2.0, 0.0, 0.0]      # 1 + 4
    v1[0, 1, 3] = -3.0                      # + 9
    assert O.kv_deviation(k1, v1, k0, v0).tolist() == [14.0]
    assert O.kv_deviation(k0, v0, k1, v1).tolist() == [14.0]      # symmetric


def test_deviation_of_rows_differing_only_in_k():
    k0, v0 = _rows()
    k1, v1 = k0.copy(), v0.copy()
    k1[0, 0, 1] = 0.5                       # 0.25
    k1[0, 1, 2] = 2.0                       # + 4
    assert O.kv_deviation(k1, v1, k0, v0).tolist() == [4.25]


def test_deviation_of_rows_differing_only_in_the_second_kv_head():
    k0, v0 = _rows(hkv=2)
    k1, v1 = k0.copy(), v0.copy()
    k1[0, 1, :] = [1.0, 1.0, 1.0, 1.0]      # 4
    v1[0, 1, :] = [0.0, 0.0, 0.0, 6.0]      # + 36
    assert O.kv_deviation(k1, v1, k0, v0).tolist() == [40.0]
    # the first head alone would give 0: the score must run over every KV head
    assert O.kv_deviation(k1[:, :1], v1[:, :1], k0[:, :1], v0[:, :1]).tolist() == [0.0]


def test_deviation_of_a_pythagorean_pair_is_the_squared_norm():
    # K differs by (3, 0, ...), V by (0, 4, ...): ||dKV|| = 5, reported squared
    k0, v0 = _rows(hkv=1, dh=2)
    k1, v1 = k0.copy(), v0.copy()
    k1[0, 0, 0] = 3.0
    v1[0, 0, 1] = 4.0
    assert O.kv_deviation(k1, v1, k0, v0).tolist() == [25.0]


def test_deviation_per_row_of_a_batch():
    k0, v0 = _rows(n=3, hkv=2, dh=2)
    k1, v1 = k0 + 1.0, v0.copy()            # row sums: 4 ones in K -> 4
    v1[1] = 2.0                             # row 1: + 4 * 4 = 16
    k1[2] = k0[2]                           # row 2: K equal, V equal -> 0
    assert O.kv_deviation(k1, v1, k0, v0).tolist() == [4.0, 20.0, 0.0]


def test_deviation_is_invariant_under_a_common_rotation():
    # the score compares post-RoPE K: a rotation R(p) applied to both sides keeps it (R orthogonal)
    rng = np.random.default_rng(3)
    a, b = rng.standard_normal((2, 5, 2, 8))
    v = rng.standard_normal((5, 2, 8))
    pos = np.arange(100, 105)
    d0 = O.kv_deviation(a, v, b, v)
    d1 = O.kv_deviation(O.rope_rotate(a, pos, 10000.0), v, O.rope_rotate(b, pos, 10000.0), v)
    np.testing.assert_allclose(d0, d1, rtol=1e-12)


def test_blend_layer_deviation_by_element_loop():
    """Brute force on a tiny layer: the deviation blend_layer reports for each candidate row is
    the sum over every KV head and every element of K and V of (fresh - fused before the
    scatter)^2, summed in a plain Python loop."""
    wl = F.get_config("tiny_gqa")
    sh = wl.shape
    W = F.layer_weights(sh, 2)
    rng = np.random.default_rng(7)
    n_ctx, n_q = 12, 3
    n = n_ctx + n_q
    sel = np.array([1, 4, 5, 9, 11, 12, 13, 14])
    h = rng.standard_normal((len(sel), sh.d_model))
    fk = rng.standard_normal((n, sh.n_kv_heads, sh.head_dim)) * 0.1
    fv = rng.standard_normal((n, sh.n_kv_heads, sh.head_dim)) * 0.1
    r = O.blend_layer(sh, W, O.F64, h, fk, fv, n_ctx, sel, n_q, 0.5)
    n_cand = len(sel) - n_q
    assert len(r["deviation"]) == n_cand
    for i in range(n_cand):
        p = sel[i]
        s = 0.0
        for g in range(sh.n_kv_heads):
            for e in range(sh.head_dim):
                s += (r["k_new"][i, g, e] - fk[p, g, e]) ** 2
                s += (r["v_new"][i, g, e] - fv[p, g, e]) ** 2
        assert r["deviation"][i] == pytest.approx(s, rel=1e-12)
    # the fresh K is post-RoPE at the row's own position, V is the plain projection
    x = O.rmsnorm(h, W["g_attn"], sh.rms_eps)
    k_pre = (x @ W["w_k"].astype(np.float64).T).reshape(len(sel), sh.n_kv_heads, sh.head_dim)
    np.testing.assert_allclose(r["k_new"], O.rope_rotate(k_pre, sel, sh.rope_base), atol=1e-12)
    np.testing.assert_allclose(r["v_new"].reshape(len(sel), -1), x @ W["w_v"].astype(np.float64).T, atol=1e-12)
    # the fused rows handed in are not modified: the score saw the cache before the scatter
    assert not np.shares_memory(r["fused_k"], fk)


# ---------------------------------------------------------------- bfloat16 rounding of the oracle
def _round_u64(a):
    """IEEE round to nearest, ties to even, of float32 bit patterns to bfloat16, worked in 64-bit
    integers: add 0x7FFF plus the lowest kept bit, then drop the low 16 bits."""
    w = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((w + 0x7FFF + ((w >> 16) & 1)) >> 16).astype(np.uint32) << 16


def test_round_bf16_known_values():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.0, 0.0, -0.0,
                  3.3895313892515355e38, 1e-40, -(1 + 2**-8)], np.float64)
    want = np.array([1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -2.0, 0.0, -0.0, 3.3895313892515355e38,
                     float(np.uint32(0x00010000).view(np.float32)), -1.0])
    got = O.round_bf16(x)
    assert got.dtype == np.float64
    assert np.array_equal(got, want.astype(np.float32).astype(np.float64))
    assert np.signbit(got[6])


@pytest.mark.parametrize("seed", range(3))
def test_round_bf16_matches_64_bit_definition(seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, 1000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    ext = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x00008000, 0x80008000, 0x7F800000], np.uint32)
    x = np.concatenate([bits, ties, ext]).view(np.float32)
    x = x[np.isfinite(x)]
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got.astype(np.float32).view(np.uint32), _round_u64(x))


def test_round_bf16_of_float64_rounds_through_float32():
    # values held in float64 are first taken to the nearest float32 (the precision the kernels
    # compute in) and then rounded to bfloat16
    rng = np.random.default_rng(11)
    x = rng.standard_normal(100_000) * 10.0 ** rng.integers(-6, 6, 100_000)
    got = O.round_bf16(x)
    assert np.array_equal(got.astype(np.float32).view(np.uint32), _round_u64(x.astype(np.float32)))
    # and only bfloat16 values come out: rounding again changes nothing
    assert np.array_equal(O.round_bf16(got), got)


def test_precision_rounds_only_in_bf16_mode():
    x = np.array([1 + 2**-8 + 2**-20, 0.1])
    assert np.array_equal(O.Precision("f64").store(x), x)
    assert np.array_equal(O.Precision("bf16").store(x), O.round_bf16(x))
    assert O.Precision.for_dtype("bf16").kind == "bf16" and O.Precision.for_dtype("f32").kind == "f64"
