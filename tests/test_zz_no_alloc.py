"""cb_blend_layer_static (the library's static workspace, no workspace argument) against
cb_blend_layer with a caller workspace: two calls in a row, the second on a smaller input
(the first call's kept rows, narrowed further), each output compared bit for bit; and a call
whose workspace would exceed the static array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import fixtures as F
from gpu_setup import bits, engine

pytestmark = pytest.mark.gpu

STATIC_BYTES = 128 << 20


def _p(t):
    return 0 if t is None else int(t.data_ptr())


def _run(eng, L, fn, layer, h, sel, cache, offs, n_query, ratio, with_dev):
    d = eng.device
    sh = eng.shape
    n_tok = int(offs[-1]) + n_query
    n_sel = len(sel)
    h_d = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(d)
    sel_d = torch.from_numpy(np.asarray(sel, np.int32)).to(d)
    offs_d = torch.tensor(list(offs), dtype=torch.int32, device=d)
    fk, fv = eng.kv_empty(n_tok), eng.kv_empty(n_tok)
    new_sel = torch.full((n_tok,), -1, dtype=torch.int32, device=d)
    new_loc = torch.full((n_tok,), -1, dtype=torch.int32, device=d)
    out = torch.zeros(n_tok, sh.n_q_heads * sh.head_dim, dtype=eng.dtype, device=d)
    dev = torch.zeros(n_tok, device=d) if with_dev else None
    args = [eng.ctx, layer, _p(h_d), _p(cache[0]), _p(cache[1]), _p(fk), _p(fv), _p(offs_d), list(offs), len(offs) - 1,
            _p(sel_d), n_sel, n_query, ratio, _p(new_sel), _p(new_loc), _p(out), _p(dev)]
    if fn is L.cb_blend_layer:
        ws = eng.workspace(n_tok, n_sel)
        n_new = fn(*args, _p(ws), ws.numel())
    else:
        n_new = fn(*args)
    eng.compute.synchronize()
    res = {"n_new": n_new, "new_sel": new_sel[:n_new].cpu().numpy(), "new_loc": new_loc[:n_new].cpu().numpy(),
           "out": bits(out[:n_new]), "fk": bits(fk), "fv": bits(fv)}
    if with_dev:
        res["dev"] = dev[: n_sel - n_query].cpu().numpy()
    return res


@pytest.mark.parametrize("cfg", ["small_bf16", "tiny"])
def test_static_workspace_matches_caller_workspace(cfg):
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import build_chunk_caches
    wl = F.get_config(cfg)
    sh = wl.shape
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    offs = [int(o) for o in F.chunk_offsets(wl)]
    n_tok = wl.n_tokens
    need = L.cb_workspace_size(eng.ctx, n_tok, n_tok)
    assert need <= STATIC_BYTES, need
    rng = np.random.default_rng(3)
    h1 = rng.standard_normal((n_tok, sh.d_model)).astype(np.float32)
    sel1 = np.arange(n_tok)

    def two_calls(fn):
        a = _run(eng, L, fn, 1, h1, sel1, cache[1], offs, wl.n_query, 0.30, True)
        sel2 = a["new_sel"]  # the kept rows: a smaller input, narrowed to 15%
        h2 = rng2.standard_normal((len(sel2), sh.d_model)).astype(np.float32)
        b = _run(eng, L, fn, 2 % sh.n_layers, h2, sel2, cache[2 % sh.n_layers], offs, wl.n_query, 0.15, False)
        return a, b

    rng2 = np.random.default_rng(4)
    st = two_calls(L.cb_blend_layer_static)
    rng2 = np.random.default_rng(4)
    ref = two_calls(L.cb_blend_layer)
    for i, (x, y) in enumerate(zip(st, ref)):
        assert x["n_new"] == y["n_new"] and x["n_new"] > wl.n_query, (i, x["n_new"], y["n_new"])
        for key in x:
            if key == "n_new":
                continue
            assert np.array_equal(x[key], y[key]), f"call {i + 1}: {key} differs"
    assert st[1]["n_new"] < st[0]["n_new"]
    eng.close()


def test_static_workspace_refuses_oversized_calls():
    from rag_kv_cache_amd import _lib as L
    from rag_kv_cache_amd.pipeline import Engine
    from gpu_setup import weights
    cfg = "small_bf16"
    wl = F.get_config(cfg)
    sh = wl.shape
    W, E = weights(cfg)
    n_tok, n_q = 8000, 100
    eng = Engine(sh, max_tokens=n_tok)
    eng.load_all(lambda l: W[l - 1], E)
    need = L.cb_workspace_size(eng.ctx, n_tok, n_tok)
    assert need > STATIC_BYTES, need  # the call below must be refused on the host
    d = eng.device
    offs = [0, n_tok - n_q]
    h = torch.zeros(n_tok, sh.d_model, device=d)
    sel = torch.arange(n_tok, dtype=torch.int32, device=d)
    offs_d = torch.tensor(offs, dtype=torch.int32, device=d)
    fk, fv = eng.kv_empty(n_tok), eng.kv_empty(n_tok)
    ck, cv = eng.kv_empty(n_tok), eng.kv_empty(n_tok)
    new_sel = torch.empty(n_tok, dtype=torch.int32, device=d)
    new_loc = torch.empty(n_tok, dtype=torch.int32, device=d)
    out = torch.empty(n_tok, sh.n_q_heads * sh.head_dim, dtype=eng.dtype, device=d)
    with pytest.raises(L.CbError) as e:
        L.cb_blend_layer_static(eng.ctx, 1, _p(h), _p(ck), _p(cv), _p(fk), _p(fv), _p(offs_d), offs, 1, _p(sel),
                                n_tok, n_q, 0.15, _p(new_sel), _p(new_loc), _p(out), 0)
    assert e.value.status == L.CB_ENOMEM
    assert "static scratch" in L.cb_last_error()
    eng.compute.synchronize()
    eng.close()
