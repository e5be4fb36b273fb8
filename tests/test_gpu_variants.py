"""GPU parity of the selection variants (KVBoost page, section on seam repair) against the
oracle: the cosine deviation score with gradual filtering, and the spatial seam set kept at
every layer.  fp32 fixture workloads, whole pipeline, the same comparisons as the default
score's pipeline test."""
import numpy as np
import pytest

import fixtures as F
import oracle as O
from parity_util import assert_close, check_selected, local_index
from gpu_setup import engine, fused_buffers, to_np, weights

pytestmark = pytest.mark.gpu


def _run(cfg, score=None, initial_sel=None, schedule=None):
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    wl = F.get_config(cfg)
    eng = engine(cfg)
    if score is not None:
        L.cb_set_score_mode(eng.ctx, score)
    cache, _ = build_chunk_caches(eng, F.chunk_tokens(wl))
    buf = make_buffers(eng, wl.n_tokens, len(wl.chunk_lens))
    fused = fused_buffers(eng, wl.n_tokens)
    res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, schedule or wl.schedule, fused,
                     cache=cache, record=True, initial_sel=initial_sel)
    eng.compute.synchronize()
    return wl, eng, fused, res, cache


def _compare(wl, fused, res, ref):
    for l, (rec, Lr) in enumerate(zip(res.records, ref["layers"])):
        n_cand = len(Lr["sel"]) - wl.n_query
        assert np.array_equal(rec.sel, Lr["sel"]), f"layer {l}: S_l differs"
        assert_close(rec.deviation, Lr["deviation"].astype(np.float32), "f32", f"deviation layer {l}")
        flips = check_selected(rec.new_sel, Lr["new_sel"], Lr["deviation"], Lr["sel"][:n_cand], Lr["k"], wl.n_query)
        assert flips == 0, f"layer {l}: near-tie flip breaks the pipeline comparison"
        assert_close(to_np(fused[l][0]), Lr["fused_k"], "f32", f"fused K layer {l}")
        assert_close(to_np(fused[l][1]), Lr["fused_v"], "f32", f"fused V layer {l}")
        assert_close(rec.out_sel, Lr["out"], "f32", f"attention out layer {l}")
        assert_close(rec.hidden_out, Lr["hidden_out"], "f32", f"hidden out layer {l}")
    assert np.array_equal(res.sel[: res.n_final].cpu().numpy(), ref["sel"])


@pytest.mark.parametrize("cfg", ["tiny", "tiny3", "tiny_gqa"])
def test_cosine_score_pipeline_matches_oracle(cfg):
    from rag_kv_cache_amd import _lib as L
    wl, eng, fused, res, _ = _run(cfg, score=L.CB_SCORE_COSINE)
    W, E = weights(cfg)
    ref = O.blended_prefill(wl.shape, W, E, F.chunk_tokens(wl), F.query_tokens(wl), wl.schedule, score="cosine")
    _compare(wl, fused, res, ref)
    # the score is really the cosine one: deviations lie in [0, 2]
    for rec in res.records:
        assert rec.deviation.min(initial=0.0) >= -1e-6 and rec.deviation.max(initial=0.0) <= 2.0 + 1e-6


@pytest.mark.parametrize("cfg", ["tiny3", "tiny_gqa"])
@pytest.mark.parametrize("window", [16, 3])
def test_seam_set_pipeline_matches_oracle(cfg, window):
    from rag_kv_cache_amd import _lib as L
    wl = F.get_config(cfg)
    offs = [int(o) for o in F.chunk_offsets(wl)]
    seam = L.cb_seam_select(offs, len(offs) - 1, wl.n_query, window)
    assert seam == O.seam_positions(offs, wl.n_query, window).tolist()
    sched = [1.0] * wl.shape.n_layers
    wl, eng, fused, res, _ = _run(cfg, initial_sel=seam, schedule=sched)
    W, E = weights(cfg)
    ref = O.blended_prefill(wl.shape, W, E, F.chunk_tokens(wl), F.query_tokens(wl), sched,
                            initial_sel=np.asarray(seam))
    _compare(wl, fused, res, ref)
    for rec in res.records:  # the set is fixed at every layer
        assert rec.sel.tolist() == seam and rec.new_sel.tolist() == seam


def test_cosine_bf16_teacher_forced():
    """bf16 shape, cosine score: per layer, the GPU's deviations and kept set against the
    oracle fed with the GPU's own inputs (bf16 rounding points emulated)."""
    from rag_kv_cache_amd import _lib as L
    cfg = "small_bf16"
    wl, eng, fused, res, cache = _run(cfg, score=L.CB_SCORE_COSINE)
    sh = wl.shape
    W, E = weights(cfg)
    prec = O.Precision("bf16")
    offs = F.chunk_offsets(wl)
    hidden = np.asarray(E[F.all_tokens(wl)], np.float64)
    for l, rec in enumerate(res.records):
        gpu_cache = [(to_np(cache[l][0])[offs[c]:offs[c + 1]], to_np(cache[l][1])[offs[c]:offs[c + 1]])
                     for c in range(len(wl.chunk_lens))]
        fk, fv = O.fuse_cache(sh, prec, gpu_cache, offs, wl.n_query)
        r = O.blend_layer(sh, W[l], prec, hidden, fk, fv, wl.n_ctx, rec.sel, wl.n_query, wl.schedule[l],
                          new_sel_override=rec.new_sel, score="cosine")
        r_own = O.blend_layer(sh, W[l], prec, hidden, fk, fv, wl.n_ctx, rec.sel, wl.n_query, wl.schedule[l],
                              score="cosine")
        n_cand = len(rec.sel) - wl.n_query
        err = np.abs(rec.deviation - r["deviation"]) - 1e-3 * np.abs(r["deviation"])
        assert err.max(initial=0.0) <= 1e-4, f"layer {l}: cosine deviation err {err.max():.2e}"
        check_selected(rec.new_sel, r_own["new_sel"], r_own["deviation"], rec.sel[:n_cand], r_own["k"], wl.n_query)
        assert_close(rec.out_sel, r["out"], "bf16", f"attention out layer {l}")
        h_ref = O.layer_rest(sh, W[l], prec, hidden, local_index(rec.sel, rec.new_sel), rec.out_sel)
        assert_close(rec.hidden_out, h_ref, "bf16", f"hidden out layer {l}")
        hidden = rec.hidden_out.astype(np.float64)
