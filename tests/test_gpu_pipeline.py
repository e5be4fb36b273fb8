"""GPU parity of the whole fused prefill against the oracle (fixture workloads small enough
for the oracle to finish in seconds; ragged chunk lengths; several GEMM/attention tiles)."""
import numpy as np
import pytest

import fixtures as F
import oracle as O
from parity_util import assert_close, check_selected, local_index
from gpu_setup import bits, engine, fused_buffers, to_np, weights

pytestmark = pytest.mark.gpu


def _gpu_run(cfg, record=True):
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    wl = F.get_config(cfg)
    eng = engine(cfg)
    chunks, q = F.chunk_tokens(wl), F.query_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = fused_buffers(eng, wl.n_tokens)
    res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                     cache=cache, record=record)
    eng.compute.synchronize()
    return wl, eng, cache, fused, res


@pytest.mark.parametrize("cfg", ["tiny", "tiny3", "tiny_gqa"])
def test_fp32_pipeline_matches_oracle(cfg):
    wl, eng, cache, fused, res = _gpu_run(cfg)
    sh = wl.shape
    W, E = weights(cfg)
    ref = O.blended_prefill(sh, W, E, F.chunk_tokens(wl), F.query_tokens(wl), wl.schedule)
    offs = F.chunk_offsets(wl)
    for l in range(sh.n_layers):  # chunk caches built on the GPU vs the oracle's
        ck = np.concatenate([ref["caches"][c][l][0] for c in range(len(wl.chunk_lens))])
        cv = np.concatenate([ref["caches"][c][l][1] for c in range(len(wl.chunk_lens))])
        assert_close(to_np(cache[l][0]), ck, "f32", f"cache K layer {l}")
        assert_close(to_np(cache[l][1]), cv, "f32", f"cache V layer {l}")
    for l, (rec, L) in enumerate(zip(res.records, ref["layers"])):
        n_cand = len(L["sel"]) - wl.n_query
        assert np.array_equal(rec.sel, L["sel"]), f"layer {l}: S_l differs"
        assert_close(rec.deviation, L["deviation"].astype(np.float32), "f32", f"deviation layer {l}")
        flips = check_selected(rec.new_sel, L["new_sel"], L["deviation"], L["sel"][:n_cand], L["k"], wl.n_query)
        assert flips == 0, f"layer {l}: near-tie flip breaks the pipeline comparison"
        assert_close(to_np(fused[l][0]), L["fused_k"], "f32", f"fused K layer {l}")
        assert_close(to_np(fused[l][1]), L["fused_v"], "f32", f"fused V layer {l}")
        assert_close(rec.out_sel, L["out"], "f32", f"attention out layer {l}")
        assert_close(rec.hidden_out, L["hidden_out"], "f32", f"hidden out layer {l}")
    assert np.array_equal(res.sel[: res.n_final].cpu().numpy(), ref["sel"])


def test_bf16_calls_teacher_forced():
    """Each layer's blend_layer and layer_rest against the oracle on the GPU's own inputs
    (bf16 rounding points emulated), so a near-tie resolved differently at one layer does not
    propagate; plus the GPU chunk caches against the oracle's."""
    cfg = "small_bf16"
    wl, eng, cache, fused, res = _gpu_run(cfg)
    sh = wl.shape
    W, E = weights(cfg)
    prec = O.Precision("bf16")
    chunks = F.chunk_tokens(wl)
    ref_caches = O.chunk_caches(sh, W, E, chunks, prec)
    offs = F.chunk_offsets(wl)
    for l in range(sh.n_layers):
        assert_close(to_np(cache[l][0]), np.concatenate([c[l][0] for c in ref_caches]), "bf16", f"cache K {l}")
        assert_close(to_np(cache[l][1]), np.concatenate([c[l][1] for c in ref_caches]), "bf16", f"cache V {l}")
    hidden = np.asarray(E[F.all_tokens(wl)], np.float64)
    flips_total = 0
    for l, rec in enumerate(res.records):
        gpu_cache = [(to_np(cache[l][0])[offs[c]:offs[c + 1]], to_np(cache[l][1])[offs[c]:offs[c + 1]])
                     for c in range(len(chunks))]
        fk, fv = O.fuse_cache(sh, prec, gpu_cache, offs, wl.n_query)
        r = O.blend_layer(sh, W[l], prec, hidden, fk, fv, wl.n_ctx, rec.sel, wl.n_query, wl.schedule[l],
                          new_sel_override=rec.new_sel)
        # the oracle's own choice on the same inputs
        r_own = O.blend_layer(sh, W[l], prec, hidden, fk, fv, wl.n_ctx, rec.sel, wl.n_query, wl.schedule[l])
        n_cand = len(rec.sel) - wl.n_query
        # rtol 1e-3 plus an absolute floor for layers where d is pure rounding noise (layer 1)
        err = np.abs(rec.deviation - r["deviation"]) - 1e-3 * np.abs(r["deviation"])
        assert err.max(initial=0.0) <= 1e-3, f"layer {l}: deviation err {err.max():.2e}"
        flips_total += check_selected(rec.new_sel, r_own["new_sel"], r_own["deviation"], rec.sel[:n_cand],
                                      r_own["k"], wl.n_query)
        assert_close(to_np(fused[l][0]), r["fused_k"], "bf16", f"fused K layer {l}")
        assert_close(to_np(fused[l][1]), r["fused_v"], "bf16", f"fused V layer {l}")
        assert_close(rec.out_sel, r["out"], "bf16", f"attention out layer {l}")
        h_ref = O.layer_rest(sh, W[l], prec, hidden, local_index(rec.sel, rec.new_sel), rec.out_sel)
        assert_close(rec.hidden_out, h_ref, "bf16", f"hidden out layer {l}")
        hidden = rec.hidden_out.astype(np.float64)
    print(f"near-tie flips: {flips_total}")


def test_repeat_runs_are_bit_identical():
    from rag_kv_cache_amd.pipeline import make_buffers, run_layers
    wl, eng, cache, fused, res = _gpu_run("small_bf16", record=False)
    a = (res.hidden[: res.n_final].cpu().numpy().copy(), [bits(f[0]) for f in fused])
    buf = make_buffers(eng, wl.n_tokens, len(wl.chunk_lens))
    fused2 = fused_buffers(eng, wl.n_tokens)
    res2 = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused2,
                      cache=cache)
    eng.compute.synchronize()
    assert res2.n_final == res.n_final
    assert np.array_equal(res2.hidden[: res2.n_final].cpu().numpy(), a[0])
    for x, y in zip(fused2, a[1]):
        assert np.array_equal(bits(x[0]), y)


def test_prefetch_path_equals_hbm_path():
    """Pinned-host cache fetched two layers ahead on the copy stream (read over PCIe and
    rotated by one kernel, at the default launch shape and at others down to one wavefront, or
    copied by the copy engine and rotated in place, or from pageable
    memory, which falls back to the copy engine), the HBM-resident cache re-rotated by copy on
    the copy stream, and re-rotated inside each cb_blend_layer, all give bit-identical results
    to the HBM-resident cache re-rotated for every layer in one launch (cb_rotate_layers).  The
    copy-engine case also runs with chunks adjacent in host memory (one copy per run)."""
    import torch
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    cfg = "small_bf16"
    wl = F.get_config(cfg)
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    from rag_kv_cache_amd import _lib as L
    cache, host = build_chunk_caches(eng, chunks, pinned_host=True)
    pageable = [[(k.clone(), v.clone()) for k, v in layer] for layer in host]  # not page-locked
    assert not pageable[0][0][0].is_pinned()
    # chunks adjacent in host memory (as consecutive chunk-store entries are): the copy path moves
    # each run of adjacent chunks in one copy; here chunks 0-1 form one run and the rest another
    runs = []
    for layer in host:
        n0 = layer[0][0].shape[0] + layer[1][0].shape[0]
        kk = [torch.cat([k for k, _ in layer[:2]]).pin_memory(), torch.cat([k for k, _ in layer[2:]]).pin_memory()]
        vv = [torch.cat([v for _, v in layer[:2]]).pin_memory(), torch.cat([v for _, v in layer[2:]]).pin_memory()]
        row, out = 0, []
        for c, (k, _) in enumerate(layer):
            part = 0 if c < 2 else 1
            r0 = row if c < 2 else row - n0
            out.append((kk[part][r0: r0 + k.shape[0]], vv[part][r0: r0 + k.shape[0]]))
            row += k.shape[0]
        runs.append(out)
    assert runs[0][1][0].data_ptr() == runs[0][0][0].data_ptr() + runs[0][0][0].numel() * runs[0][0][0].element_size()
    outs = []
    shapes = {"prefetch_3x192x2": (3, 192, 2), "prefetch_1x64x1": (1, 64, 1), "prefetch_40x1024x4": (40, 1024, 4)}
    for mode in ("hbm", "prefetch", "prefetch_copy", "prefetch_copy_runs", "prefetch_pageable", "hbm_copy_stream",
                 "hbm_per_layer", *shapes):
        buf = make_buffers(eng, wl.n_tokens, len(chunks))
        fused = fused_buffers(eng, wl.n_tokens)
        pre = mode.startswith("prefetch")
        L.cb_set_fetch_mode(eng.ctx, L.CB_FETCH_COPY if mode.startswith("prefetch_copy") else L.CB_FETCH_KERNEL)
        L.cb_set_fetch_launch(eng.ctx, *shapes.get(mode, (0, 0, 0)))
        hc = {"prefetch_pageable": pageable, "prefetch_copy_runs": runs}.get(mode, host)
        res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                         cache=None if pre else cache, host_cache=hc if pre else None,
                         rotate_on_copy_stream=mode == "hbm_copy_stream", batch_rotation=mode != "hbm_per_layer")
        eng.compute.synchronize()
        L.cb_set_fetch_mode(eng.ctx, L.CB_FETCH_KERNEL)
        L.cb_set_fetch_launch(eng.ctx, 0, 0, 0)
        outs.append((res.hidden[: res.n_final].cpu().numpy().copy(), res.sel[: res.n_final].cpu().numpy().copy(),
                     [(bits(k), bits(v)) for k, v in fused]))
    h0, s0, f0 = outs[0]
    for h1, s1, f1 in outs[1:]:
        assert np.array_equal(s0, s1)
        assert np.array_equal(h0, h1)
        for (a, b), (c, d) in zip(f0, f1):
            assert np.array_equal(a, c) and np.array_equal(b, d)


@pytest.mark.parametrize("sched", [(1.0, 1.0, 1.0), (1.0, 0.0, 0.0)])
def test_special_schedules(sched):
    """Ratio 1 everywhere = full prefill of the whole prompt; ratio 0 keeps only query rows
    and leaves the re-rotated cache in place."""
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    cfg = "tiny_gqa"
    wl = F.get_config(cfg)
    sh = wl.shape
    W, E = weights(cfg)
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = fused_buffers(eng, wl.n_tokens)
    res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, list(sched), fused,
                     cache=cache, record=True)
    eng.compute.synchronize()
    if sched[1] == 1.0:
        full = O.full_prefill(sh, W, E, F.all_tokens(wl))
        for l in range(sh.n_layers):
            assert_close(to_np(fused[l][0]), full["k"][l], "f32", f"K layer {l}")
            assert_close(to_np(fused[l][1]), full["v"][l], "f32", f"V layer {l}")
        assert_close(res.hidden[: res.n_final].cpu().numpy(), full["hidden"][-1], "f32", "hidden")
    else:
        assert res.records[1].new_sel.tolist() == list(range(wl.n_ctx, wl.n_tokens))
        offs = F.chunk_offsets(wl)
        for l in (2,):  # from layer 3 on no context row is recomputed: the re-rotated cache stays
            rot = O.fuse_cache(sh, O.F64, [(to_np(cache[l][0])[offs[c]:offs[c + 1]],
                                            to_np(cache[l][1])[offs[c]:offs[c + 1]]) for c in range(3)],
                               offs, wl.n_query)
            assert_close(to_np(fused[l][0])[: wl.n_ctx], rot[0][: wl.n_ctx], "f32", "rotated K")
            assert np.array_equal(bits(fused[l][1][: wl.n_ctx]), bits(cache[l][1]))


def test_many_chunks_and_layers_batched_paths():
    """More than 64 chunks (the fetch kernel then runs in batches of 64) and more than 64 layers
    (cb_rotate_layers then launches per 64 layers): both batched paths give bit-identical results
    to the per-layer paths (copy engine + rotation inside cb_blend_layer)."""
    from dataclasses import replace
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, make_buffers, run_layers
    base = F.get_config("tiny")
    sh = replace(base.shape, name="tiny-deep", n_layers=66, d_model=128, ffn_dim=256, vocab=500)
    wl = F.Workload("many_chunks", sh, (4,) * 70 + (9,), 7, (1.0,) + (0.3,) * 65)
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    eng = Engine(sh, max_tokens=wl.n_tokens + 8)
    eng.load_all(lambda l: W[l - 1], F.embedding(sh))
    chunks = F.chunk_tokens(wl)
    cache, host = build_chunk_caches(eng, chunks, pinned_host=True)
    outs = []
    for mode in ("hbm_batched", "hbm_per_layer", "prefetch_kernel", "prefetch_copy"):
        L.cb_set_fetch_mode(eng.ctx, L.CB_FETCH_COPY if mode == "prefetch_copy" else L.CB_FETCH_KERNEL)
        buf = make_buffers(eng, wl.n_tokens, len(chunks))
        fused = fused_buffers(eng, wl.n_tokens)
        pre = mode.startswith("prefetch")
        res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                         cache=None if pre else cache, host_cache=host if pre else None,
                         batch_rotation=mode == "hbm_batched")
        eng.compute.synchronize()
        outs.append((res.hidden[: res.n_final].cpu().numpy().copy(), [(bits(k), bits(v)) for k, v in fused]))
    L.cb_set_fetch_mode(eng.ctx, L.CB_FETCH_KERNEL)
    h0, f0 = outs[0]
    for h1, f1 in outs[1:]:
        assert np.array_equal(h0, h1)
        for (a, b), (c, d) in zip(f0, f1):
            assert np.array_equal(a, c) and np.array_equal(b, d)
    eng.close()


@pytest.mark.parametrize("weights,schedule", [("bf16", (1.0, 0.30, 0.15, 0.15)), ("int8", (1.0, 0.30, 0.15, 0.15)),
                                              ("bf16", (1.0, 0.30, 0.0, 0.0))])
def test_kv_scatter_in_product_epilogue_gives_the_scatter_kernels_bits(weights, schedule):
    """With no deviation asked for (a run that records nothing), a layer that keeps every
    candidate (layer 1 at ratio 1, layer 4 at an unchanged 15%, or layer 4 after layer 3 kept
    only the query rows) writes its fresh K/V into the fused cache from the K/V product's
    epilogue, and the kept set with it, instead of running the deviation + scatter kernel, whose
    deviation would select nothing.  On the Qwen shape's first four layers (unsplit MFMA tiles:
    5184 rows at layer 1, 832 at layer 4; split-K with the epilogue in the reduce: the 64 query
    rows at layer 4), with bf16 or int8 weights, the step gives the same bits as the recorded run,
    which asks for deviations and takes the kernel."""
    from dataclasses import replace
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import Engine, build_chunk_caches, make_buffers, run_layers
    base = F.get_config("qwen")
    sh = replace(base.shape, name="qwen-4-layers", n_layers=4)
    wl = replace(base, shape=sh, schedule=schedule)
    eng = Engine(sh, max_tokens=wl.n_tokens + 8)
    if weights == "bf16":
        W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
        eng.load_all(lambda l: W[l - 1], F.embedding(sh))
    else:
        for l in range(sh.n_layers):
            eng.load_layer_int8(l, F.layer_weights_int8(sh, l + 1))
        eng.load_embedding(F.embedding(sh))
    cache, _ = build_chunk_caches(eng, F.chunk_tokens(wl))
    outs = []
    for record in (True, False):
        buf = make_buffers(eng, wl.n_tokens, len(wl.chunk_lens))
        fused = [(eng.kv_empty(wl.n_tokens), eng.kv_empty(wl.n_tokens)) for _ in range(sh.n_layers)]
        L.cb_profile_enable(eng.ctx, True)
        res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                         cache=cache, record=record)
        eng.compute.synchronize()
        L.cb_profile_enable(eng.ctx, False)
        _, scatter_launches, _ = L.cb_profile_read(eng.ctx, L.CB_K_DEV_SCATTER)
        outs.append((res.hidden[: res.n_final].cpu().numpy().copy(), res.sel[: res.n_final].cpu().numpy().copy(),
                     [(bits(k), bits(v)) for k, v in fused], scatter_launches))
    (h0, s0, f0, n0), (h1, s1, f1, n1) = outs
    assert n0 == 4 and n1 == 2, (n0, n1)  # layers 2 and 3 narrow the set: their deviation selects
    assert np.array_equal(s0, s1)
    assert np.array_equal(h0, h1)
    for (a, b), (c, d) in zip(f0, f1):
        assert np.array_equal(a, c) and np.array_equal(b, d)
    eng.close()
