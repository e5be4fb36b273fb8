"""A whole blended prefill captured as a HIP graph: every replay must reproduce the eager
run bit for bit, also with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import fixtures as F
from gpu_setup import bits, engine, fused_buffers

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    from rag_kv_cache_amd.pipeline import build_chunk_caches, capture_step, make_buffers, run_layers
    cfg = "small_bf16"
    wl = F.get_config(cfg)
    eng = engine(cfg)
    chunks = F.chunk_tokens(wl)
    cache, _ = build_chunk_caches(eng, chunks)
    toks, offs = F.all_tokens(wl), F.chunk_offsets(wl)
    buf = make_buffers(eng, wl.n_tokens, len(chunks))
    fused = fused_buffers(eng, wl.n_tokens)

    def step(upload=False):
        return run_layers(eng, buf, toks, offs, wl.n_query, wl.schedule, fused, cache=cache, upload_inputs=upload)

    res = step(upload=True)
    eng.compute.synchronize()
    n = res.n_final
    ref_h = res.hidden[:n].cpu().numpy().copy()
    ref_f = [bits(k) for k, _ in fused]
    g = capture_step(eng, step)
    for rep in range(3):
        for k, v in fused:  # poison outputs so that a replay that skipped work is caught
            k.fill_(3.0)
            v.fill_(-3.0)
        res.hidden.fill_(0.5)
        torch.cuda.synchronize()
        with torch.cuda.stream(eng.compute):
            g.replay()
        eng.compute.synchronize()
        assert np.array_equal(res.hidden[:n].cpu().numpy(), ref_h), f"replay {rep}: hidden rows differ"
        for l, (k, _) in enumerate(fused):
            assert np.array_equal(bits(k), ref_f[l]), f"replay {rep}: fused K of layer {l} differs"
        step()  # eager work between replays
        eng.compute.synchronize()
        assert np.array_equal(res.hidden[:n].cpu().numpy(), ref_h)
