"""GPU tests of the C ABI's host-side contract: status codes, the fetch/synchronize state
machine, argument validation and edge sizes (the kernels must not run on bad input)."""
import numpy as np
import pytest
import torch

import fixtures as F
import oracle as O
from gpu_setup import engine, fused_buffers, to_np, weights
from parity_util import assert_close

pytestmark = pytest.mark.gpu


def _p(t):
    return 0 if t is None else int(t.data_ptr())


@pytest.fixture(scope="module")
def tiny():
    eng = engine("tiny")
    wl = F.get_config("tiny")
    yield eng, wl
    eng.close()


def _blend(eng, wl, l=0, n_sel=None, n_query=None, ratio=0.5, ws_bytes=None, offs=None, fused=None, cached=None):
    from rag_kv_cache_amd import _lib as L
    n_tok = wl.n_tokens
    offs = list(F.chunk_offsets(wl)) if offs is None else offs
    d = eng.device
    h = torch.zeros(n_tok, wl.shape.d_model, device=d) + 0.1
    sel = torch.arange(n_tok, dtype=torch.int32, device=d)
    offs_d = torch.tensor(offs, dtype=torch.int32, device=d)
    fk, fv = fused if fused else (eng.kv_empty(n_tok), eng.kv_empty(n_tok))
    new_sel = torch.empty(n_tok, dtype=torch.int32, device=d)
    new_loc = torch.empty(n_tok, dtype=torch.int32, device=d)
    out = torch.empty(n_tok, wl.shape.n_q_heads * wl.shape.head_dim, device=d)
    ws = eng.workspace(n_tok, n_tok)
    ck, cv = cached if cached else (None, None)
    return L.cb_blend_layer(eng.ctx, l, _p(h), _p(ck), _p(cv), _p(fk), _p(fv), _p(offs_d), offs, len(offs) - 1,
                            _p(sel), n_tok if n_sel is None else n_sel, wl.n_query if n_query is None else n_query,
                            ratio, _p(new_sel), _p(new_loc), _p(out), 0, _p(ws),
                            ws.numel() if ws_bytes is None else ws_bytes)


def test_status_codes(tiny):
    from rag_kv_cache_amd import _lib as L
    eng, wl = tiny
    with pytest.raises(L.CbError) as e:
        _blend(eng, wl, l=5)
    assert e.value.status == L.CB_EINVAL
    with pytest.raises(L.CbError) as e:
        _blend(eng, wl, n_sel=10, n_query=20)
    assert e.value.status == L.CB_ESHAPE
    with pytest.raises(L.CbError) as e:
        _blend(eng, wl, ws_bytes=16)
    assert e.value.status == L.CB_ENOMEM
    with pytest.raises(L.CbError) as e:
        _blend(eng, wl, offs=[0, 200, 100])
    assert e.value.status == L.CB_EINVAL
    with pytest.raises(L.CbError) as e:
        _blend(eng, wl, ratio=float("nan"))
    assert e.value.status == L.CB_EINVAL
    with pytest.raises(L.CbError) as e:
        L.cb_workspace_size(eng.ctx, 10, 20)
    assert e.value.status == L.CB_ESHAPE
    assert "n_sel_max" in L.cb_last_error()
    for bad in ((0, 256, 1), (8, 100, 1), (8, 2048, 1), (8, 256, 3), (2000, 64, 1), (0, 0, 1)):
        with pytest.raises(L.CbError) as e:
            L.cb_set_fetch_launch(eng.ctx, *bad)
        assert e.value.status == L.CB_EINVAL
    with pytest.raises(L.CbError) as e:
        L.cb_set_fetch_mode(eng.ctx, 7)
    assert e.value.status == L.CB_EINVAL
    L.cb_set_fetch_launch(eng.ctx, 0, 0, 0)
    assert _blend(eng, wl, ratio=0.3) == 77 + wl.n_query
    assert _blend(eng, wl, ratio=5.0) == wl.n_tokens          # k clamped to the candidates
    assert _blend(eng, wl, ratio=0.0) == wl.n_query
    eng.compute.synchronize()


def test_fetch_synchronize_state_machine(tiny):
    from rag_kv_cache_amd import _lib as L
    eng, wl = tiny
    s = wl.shape
    offs = list(F.chunk_offsets(wl))
    hk = [torch.zeros(n, s.n_kv_heads, s.head_dim, pin_memory=True) for n in wl.chunk_lens]
    hv = [torch.zeros(n, s.n_kv_heads, s.head_dim, pin_memory=True) for n in wl.chunk_lens]
    fk, fv = eng.kv_empty(wl.n_tokens), eng.kv_empty(wl.n_tokens)
    offs_d = torch.tensor(offs, dtype=torch.int32, device=eng.device)
    L.cb_fetch_layer(eng.ctx, 1, [_p(t) for t in hk], [_p(t) for t in hv], offs, len(offs) - 1, _p(offs_d),
                     _p(fk), _p(fv))
    with pytest.raises(L.CbError) as e:  # fetched twice without synchronize
        L.cb_fetch_layer(eng.ctx, 1, [_p(t) for t in hk], [_p(t) for t in hv], offs, len(offs) - 1, _p(offs_d),
                         _p(fk), _p(fv))
    assert e.value.status == L.CB_ESTATE
    with pytest.raises(L.CbError) as e:  # the device variant is subject to the same state machine
        L.cb_fetch_layer_device(eng.ctx, 1, _p(fk), _p(fv), offs, len(offs) - 1, _p(offs_d), _p(fk), _p(fv))
    assert e.value.status == L.CB_ESTATE
    with pytest.raises(L.CbError) as e:  # blend before synchronize
        _blend(eng, wl, l=1, fused=(fk, fv), cached=(None, None))
    assert e.value.status == L.CB_ESTATE
    with pytest.raises(L.CbError) as e:  # the batched position update may not overwrite a pending fetch
        L.cb_rotate_layers(eng.ctx, 1, [_p(fk)], [_p(fv)], offs, len(offs) - 1, _p(offs_d), [_p(fk)], [_p(fv)])
    assert e.value.status == L.CB_ESTATE
    with pytest.raises(L.CbError) as e:  # layers outside the model
        L.cb_rotate_layers(eng.ctx, 1, [_p(fk)] * 2, [_p(fv)] * 2, offs, len(offs) - 1, _p(offs_d), [_p(fk)] * 2,
                           [_p(fv)] * 2)
    assert e.value.status == L.CB_EINVAL
    with pytest.raises(L.CbError) as e:  # K aliased, V not
        L.cb_rotate_layers(eng.ctx, 0, [_p(fk)], [_p(hk[0])], offs, len(offs) - 1, _p(offs_d), [_p(fk)], [_p(fv)])
    assert e.value.status == L.CB_EINVAL
    L.cb_synchronize(eng.ctx, 1)
    assert _blend(eng, wl, l=1, fused=(fk, fv), cached=(None, None)) > 0
    L.cb_synchronize(eng.ctx, 1)  # no pending fetch: no-op
    eng.compute.synchronize()


def test_delayed_copy_stream_does_not_change_results():
    """The compute stream waits for the layer's copy event: stalling the copy stream behind a
    large transfer must not change what the blend reads."""
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    cfg = "small_bf16"
    wl = F.get_config(cfg)
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    cache, host = build_chunk_caches(eng, chunks, pinned_host=True)
    results = []
    for delay in (False, True):
        buf = make_buffers(eng, wl.n_tokens, len(chunks))
        fused = fused_buffers(eng, wl.n_tokens)
        for k, v in fused:  # poison: anything not fetched would show up
            k.fill_(7.0)
            v.fill_(-7.0)
        eng.compute.synchronize()
        if delay:
            big_h = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
            big_d = torch.empty(256 << 20, dtype=torch.uint8, device=eng.device)
            with torch.cuda.stream(eng.copy):
                for _ in range(4):
                    big_d.copy_(big_h, non_blocking=True)
        res = run_layers(eng, buf, F.all_tokens(wl), F.chunk_offsets(wl), wl.n_query, wl.schedule, fused,
                         host_cache=host)
        eng.compute.synchronize()
        eng.copy.synchronize()
        results.append(res.hidden[: res.n_final].cpu().numpy().copy())
    assert np.array_equal(results[0], results[1])
    assert np.isfinite(results[0]).all()


def test_single_chunk_at_offset_zero_is_exact_prefix():
    """One chunk at offset 0: its cache is the exact prefix KV, so the deviation is ~0 and the
    query rows' outputs equal a full prefill (any schedule)."""
    from rag_kv_cache_amd.pipeline import build_chunk_caches, make_buffers, run_layers
    cfg = "tiny3"
    wl = F.get_config(cfg)
    sh = wl.shape
    W, E = weights(cfg)
    eng = engine(cfg)
    chunk = F.chunk_tokens(wl)[0]
    q = F.query_tokens(wl)
    cache, _ = build_chunk_caches(eng, [chunk])
    n = len(chunk)
    n_tok = n + len(q)
    buf = make_buffers(eng, n_tok, 1)
    fused = fused_buffers(eng, n_tok)
    res = run_layers(eng, buf, np.concatenate([chunk, q]), [0, n], len(q), wl.schedule, fused, cache=cache,
                     record=True)
    eng.compute.synchronize()
    full = O.full_prefill(sh, W, E, np.concatenate([chunk, q]))
    for rec in res.records:
        assert np.abs(rec.deviation).max(initial=0.0) < 1e-9
    assert_close(res.hidden[: res.n_final].cpu().numpy()[-len(q):], full["hidden"][-1][n:], "f32", "query rows")


def test_empty_and_degenerate_sizes(tiny):
    """n_sel = 0 and n_new = 0 enqueue nothing; no context (n_chunks = 0) works as a plain prefill."""
    from rag_kv_cache_amd import _lib as L
    eng, wl = tiny
    d = eng.device
    ws = eng.workspace(wl.n_tokens, wl.n_tokens)
    z = torch.zeros(8, dtype=torch.int32, device=d)
    n = L.cb_blend_layer(eng.ctx, 0, 0, 0, 0, _p(ws), _p(ws), 0, [0], 0, 0, 0, 0, 0.5, _p(z), _p(z), _p(ws), 0,
                         _p(ws), ws.numel())
    assert n == 0
    L.cb_layer_rest(eng.ctx, 0, _p(ws), 0, _p(z), 0, _p(ws), _p(ws[1024:]), _p(ws), ws.numel())
    L.cb_embed(eng.ctx, _p(z), 0, _p(eng.emb), _p(ws))
    # context rows only, no query rows, ratio keeps 0 of them -> nothing kept, nothing attended
    assert _blend(eng, wl, n_query=0, n_sel=wl.n_ctx, ratio=0.0) == 0
    eng.compute.synchronize()


def test_topk_ties_take_lowest_positions(tiny):
    """Gradual filtering with exact ties: a cache equal to the fresh K/V gives deviation 0 at
    every row except a chosen set D, whose rows get distinct positive deviations; with k = |D| +
    20 the kept set is D, the 20 lowest positions outside D, and every query row (ascending)."""
    from rag_kv_cache_amd import _lib as L
    eng, wl = tiny
    s = wl.shape
    n_tok, n_q = wl.n_tokens, wl.n_query
    n_ctx = n_tok - n_q
    offs = [0, n_ctx]  # one chunk at offset 0: the position update is the identity
    d = eng.device
    torch.manual_seed(0)
    h = torch.randn(n_tok, s.d_model, device=d) * 0.5
    sel = torch.arange(n_tok, dtype=torch.int32, device=d)
    offs_d = torch.tensor(offs, dtype=torch.int32, device=d)
    new_sel = torch.empty(n_tok, dtype=torch.int32, device=d)
    new_loc = torch.empty(n_tok, dtype=torch.int32, device=d)
    out = torch.empty(n_tok, s.n_q_heads * s.head_dim, device=d)
    dev = torch.empty(n_tok, device=d)
    ws = eng.workspace(n_tok, n_tok)

    def blend(cache, fk, fv, ratio):
        n = L.cb_blend_layer(eng.ctx, 1, _p(h), _p(cache[0]), _p(cache[1]), _p(fk), _p(fv), _p(offs_d), offs, 1,
                             _p(sel), n_tok, n_q, ratio, _p(new_sel), _p(new_loc), _p(out), _p(dev), _p(ws),
                             ws.numel())
        eng.compute.synchronize()
        return n

    fk, fv = eng.kv_empty(n_tok), eng.kv_empty(n_tok)
    blend((None, None), fk, fv, 1.0)  # every row recomputed: fk, fv hold the fresh K/V
    rng = np.random.default_rng(5)
    D = np.sort(rng.choice(n_ctx, size=60, replace=False))
    ck, cv = fk.clone(), fv.clone()
    bump = torch.tensor(np.linspace(0.05, 3.0, len(D)), dtype=torch.float32, device=d)
    ck[torch.from_numpy(D).to(d)] += bump[:, None, None]
    k = len(D) + 20
    fk2, fv2 = eng.kv_empty(n_tok), eng.kv_empty(n_tok)
    n_new = blend((ck, cv), fk2, fv2, k / n_ctx)
    assert n_new == k + n_q
    devs = dev[:n_ctx].cpu().numpy()
    outside = np.setdiff1d(np.arange(n_ctx), D)
    assert np.all(devs[outside] == 0.0) and np.all(devs[D] > 0.0)
    expect = np.concatenate([np.sort(np.concatenate([D, outside[:20]])), np.arange(n_ctx, n_tok)])
    assert np.array_equal(new_sel[:n_new].cpu().numpy(), expect)
    assert np.array_equal(new_loc[:n_new].cpu().numpy(), expect)  # sel is the identity here
