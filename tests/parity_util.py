"""Comparison helpers for GPU-vs-oracle parity tests (no GPU needed to import)."""
from __future__ import annotations

import numpy as np

# Tolerances: fp32 configurations 1e-5; bf16 configurations max-abs 2e-2 / rel 1e-2,
# applied per element as |gpu - ref| <= atol + rtol * |ref|.
TOL = {"f32": dict(atol=1e-5, rtol=1e-5), "bf16": dict(atol=2e-2, rtol=1e-2)}
# Rows whose deviation lies within this relative band of the k-th largest one may be
# chosen either way (the two sides round differently).
TIE_BAND = 1e-3


def assert_close(got, ref, dtype: str, what: str = "") -> float:
    """|got - ref| <= atol + rtol |ref| element by element.  Returns the largest share of that
    bound any element uses (0 = equal, 1 = at the bar)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    t = TOL[dtype]
    err = np.abs(got - ref)
    bound = t["atol"] + t["rtol"] * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - t["rtol"] * np.abs(ref)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance {t}; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r}; max abs err {err.max():.3e}")
    return float((err / bound).max(initial=0.0))


def check_selected(gpu_new, ref_new, ref_dev, cand_pos, k, n_query):
    """Selected sets agree except for rows whose deviation is within TIE_BAND of the k-th
    largest (reference values).  cand_pos: positions of the candidate rows (same order as
    ref_dev).  Returns the number of tie-band rows that differ."""
    gpu_new = np.asarray(gpu_new)
    ref_new = np.asarray(ref_new)
    assert len(gpu_new) == len(ref_new) == k + n_query, (len(gpu_new), len(ref_new), k, n_query)
    assert np.all(np.diff(gpu_new) > 0), "kept positions not ascending"
    assert np.array_equal(gpu_new[k:], ref_new[k:]), "query rows differ"
    if k == 0 or k == len(cand_pos):
        assert np.array_equal(gpu_new, ref_new)
        return 0
    d = np.asarray(ref_dev, np.float32).astype(np.float64)
    dk = np.sort(d)[::-1][k - 1]
    band = np.abs(d - dk) <= TIE_BAND * max(abs(dk), 1e-30)
    must = set(np.asarray(cand_pos)[(d > dk) & ~band].tolist())
    allowed = must | set(np.asarray(cand_pos)[band].tolist())
    g = set(gpu_new[:k].tolist())
    assert must <= g, f"rows clearly above the k-th deviation missing: {sorted(must - g)[:10]}"
    assert g <= allowed, f"rows clearly below the k-th deviation selected: {sorted(g - allowed)[:10]}"
    return len(g ^ set(ref_new[:k].tolist())) // 2


def local_index(sel, new_sel):
    pos = {int(p): i for i, p in enumerate(np.asarray(sel))}
    return np.array([pos[int(p)] for p in np.asarray(new_sel)], dtype=np.int64)
