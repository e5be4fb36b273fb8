"""Shared set-up for GPU tests: engines for fixture workloads, oracle caches, runs."""
from __future__ import annotations

import functools

import numpy as np

import fixtures as F


@functools.lru_cache(maxsize=None)
def weights(cfg: str):
    wl = F.get_config(cfg)
    sh = wl.shape
    return [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)], F.embedding(sh)


def engine(cfg: str, max_tokens: int = 0):
    from rag_kv_cache_amd.pipeline import Engine
    wl = F.get_config(cfg)
    W, E = weights(cfg)
    eng = Engine(wl.shape, max_tokens=max_tokens or wl.n_tokens + 8)
    eng.load_all(lambda l: W[l - 1], E)
    return eng


def fused_buffers(eng, n_tok):
    return [(eng.kv_empty(n_tok), eng.kv_empty(n_tok)) for _ in range(eng.shape.n_layers)]


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def bits(t):
    """Raw element bits of a device tensor (bf16 has no numpy dtype)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().copy()
    return t.cpu().numpy().copy()
