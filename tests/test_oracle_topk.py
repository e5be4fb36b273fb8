"""Pins of the oracle's gradual-filtering selection (CacheBlend explainer, "Gradual
filtering"): the kept set is the k rows of largest deviation, ties to the lower
position, against exhaustive brute force; and the k rounding rule."""
import itertools
import math

import numpy as np
import pytest

import oracle as O


def _brute_topk(d, k):
    """Row j is kept iff fewer than k rows beat it; a row beats j if its value is larger,
    or equal with a lower index."""
    d = np.asarray(d, np.float32)
    keep = []
    for j in range(len(d)):
        beats = sum(1 for i in range(len(d)) if d[i] > d[j] or (d[i] == d[j] and i < j))
        if beats < k:
            keep.append(j)
    return np.array(keep, dtype=np.int64)


def test_topk_exhaustive_with_ties():
    # every assignment of 3 distinct levels to n <= 7 rows, every k
    for n in range(0, 8):
        for vals in itertools.product([0.0, 1.0, 2.5], repeat=n) if n <= 6 else [
                tuple(np.random.default_rng(n).choice([0.0, 1.0, 2.5], n))]:
            for k in range(0, n + 1):
                got = O.topk_select(np.array(vals), k)
                np.testing.assert_array_equal(got, _brute_topk(vals, k))


def test_topk_random_against_brute():
    rng = np.random.default_rng(11)
    for trial in range(200):
        n = int(rng.integers(1, 13))
        d = np.round(rng.random(n) * 4) / 4  # quantised -> many ties
        k = int(rng.integers(0, n + 1))
        np.testing.assert_array_equal(O.topk_select(d, k), _brute_topk(d, k))


def test_topk_decides_in_float32():
    # two values distinct in float64 but equal in float32 tie -> lower index wins
    d = np.array([1.0, 1.0 + 1e-12, 0.5])
    np.testing.assert_array_equal(O.topk_select(d, 1), [0])


@pytest.mark.parametrize("ratio,n_ctx,k", [
    (0.30, 256, 77), (0.15, 256, 38), (0.30, 5120, 1536), (0.15, 5120, 768),
    (0.10, 3840, 384), (0.15, 3840, 576), (0.20, 3840, 768), (0.15, 4096, 614),
    (0.15, 16384, 2458), (0.0, 5120, 0), (1.0, 5120, 5120)])
def test_k_rounding(ratio, n_ctx, k):
    assert O.k_for_ratio(ratio, n_ctx, n_ctx) == k
    assert k == math.floor(ratio * n_ctx + 0.5)


def test_k_clamped_to_candidates():
    assert O.k_for_ratio(0.3, 5120, 100) == 100
    assert O.k_for_ratio(-0.1, 5120, 100) == 0
