"""Seeded synthetic model weights, token ids and chunk layouts.

The pages measure on trained Mistral-7B / Yi-34B / Llama-70B models and on QA and
summarisation datasets, none of which exist here.  These generators stand in for
them with random-init weights of the same shapes and uniform random token ids,
laid out as retrieved chunks followed by a user query (CacheBlend explainer,
"Background & Motivation": system prompt + retrieved documents + user query; the
workloads here omit the system prompt).

Seeds: numpy SeedSequence([SEED, stream, i, j]) with
  stream 1 = weights   (i = decoder layer, 1-based; i = 0 holds the embedding),
                       (j = 0 q, 1 k, 2 v, 3 o, 4 gate, 5 up, 6 down)
  stream 2 = chunk tokens (i = chunk index)
  stream 3 = query tokens
  stream 4 = the cache perturbation used by literal layer-1 ranking tests
                       (i = layer, j = 0 for K, 1 for V).
Weights are standard_normal(float32) * 0.02; for bf16 shapes they are then
rounded to the nearest bfloat16 (ties to even) so every consumer sees the same
bf16 numbers.  RMSNorm gains are ones.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Tuple

import numpy as np

SEED = 1234
_STREAM_WEIGHTS, _STREAM_CHUNK, _STREAM_QUERY, _STREAM_PERTURB = 1, 2, 3, 4
_TENSOR_ID = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    dtype: str  # "f32" or "bf16": element type of weights, K/V, Q and attention output
    rope_base: float = 10000.0
    rms_eps: float = 1e-6


@dataclass(frozen=True)
class Workload:
    """A prompt of independently cached chunks followed by a query, plus the
    per-layer recompute ratio schedule (entry l-1 is the ratio used at layer l)."""
    name: str
    shape: ModelShape
    chunk_lens: Tuple[int, ...]
    n_query: int
    schedule: Tuple[float, ...]
    note: str = ""

    @property
    def n_ctx(self) -> int:
        return int(sum(self.chunk_lens))

    @property
    def n_tokens(self) -> int:
        return self.n_ctx + self.n_query


def _sched(n_layers: int, *stages: float) -> Tuple[float, ...]:
    """Layer 1 recomputes every row; the given stages follow; the last stage repeats."""
    s = [1.0] + list(stages)
    s = s[:n_layers]
    while len(s) < n_layers:
        s.append(stages[-1])
    return tuple(s)


TINY = ModelShape("tiny", 2, 256, 4, 4, 64, 1024, 1000, "f32")
TINY3 = replace(TINY, name="tiny3", n_layers=3)
TINY_GQA = replace(TINY, name="tiny_gqa", n_layers=3, n_kv_heads=2)
QWEN = ModelShape("qwen2.5-1.5b", 28, 1536, 12, 2, 128, 8960, 151936, "bf16")
MISTRAL = ModelShape("mistral-7b", 32, 4096, 32, 8, 128, 14336, 32000, "bf16")
YI = ModelShape("yi-34b", 60, 7168, 56, 8, 128, 20480, 64000, "bf16")
L70 = ModelShape("llama-70b", 80, 8192, 64, 8, 128, 28672, 32000, "bf16")
# bf16 shapes small enough for the oracle to run whole pipelines in seconds.
SMALL_BF16 = ModelShape("small-bf16", 3, 512, 8, 2, 128, 1024, 2000, "bf16")

CONFIGS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, (128, 128), 32, _sched(2, 0.30),
                     "2 layers; layer 2 scores all context rows and keeps 30%"),
    "tiny3": Workload("tiny3", TINY3, (128, 128), 32, _sched(3, 0.30, 0.15),
                      "3-layer variant so that the 30% -> 15% narrowing has a layer"),
    "tiny_gqa": Workload("tiny_gqa", TINY_GQA, (96, 128, 61), 19, _sched(3, 0.30, 0.15),
                         "ragged chunks and a GQA group of 2"),
    "small_bf16": Workload("small_bf16", SMALL_BF16, (200, 256, 131), 45, _sched(3, 0.30, 0.15),
                           "bf16 pipeline at sizes the oracle finishes in seconds, ragged chunks"),
    "qwen": Workload("qwen", QWEN, (512,) * 10, 64, _sched(28, 0.30, 0.15),
                     "Qwen2.5-1.5B-shaped, 10 x 512-token chunks + 64-token query, 30% -> 15%"),
    "mistral_r10": Workload("mistral_r10", MISTRAL, (640,) * 6, 256, _sched(32, 0.10)),
    "mistral_r15": Workload("mistral_r15", MISTRAL, (640,) * 6, 256, _sched(32, 0.15)),
    "mistral_r20": Workload("mistral_r20", MISTRAL, (640,) * 6, 256, _sched(32, 0.20)),
    "yi_r15": Workload("yi_r15", YI, (480,) * 8, 256, _sched(60, 0.15)),
    "l70_4k": Workload("l70_4k", L70, (512,) * 8, 256, _sched(80, 0.15)),
    "l70_16k": Workload("l70_16k", L70, (512,) * 32, 256, _sched(80, 0.15)),
}


def get_config(name: str) -> Workload:
    return CONFIGS[name]


def rng(stream: int, i: int = 0, j: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, stream, i, j])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if not np.isfinite(u.view(np.float32)).all():
        w = u.astype(np.uint64)
        return ((w + 0x7FFF + ((w >> 16) & 1)) >> 16).astype(np.uint16)
    # finite inputs: u + 0x8000 <= 0xFF807FFF, so the sum fits in 32 bits
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """float32 array whose values are the bfloat16 roundings of `a`."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    if not np.isfinite(u.view(np.float32)).all():
        return (to_bf16_bits(a).astype(np.uint32) << 16).view(np.float32)
    r = (u >> 16) & 1
    r += 0x7FFF
    u += r
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _draw(shape: ModelShape, i: int, j: int, dims: Tuple[int, int]) -> np.ndarray:
    w = rng(_STREAM_WEIGHTS, i, j).standard_normal(dims, dtype=np.float32)
    w *= np.float32(0.02)
    if shape.dtype == "bf16":
        w = to_bf16_values(w)
    return w


def layer_weights(shape: ModelShape, layer: int) -> Dict[str, np.ndarray]:
    """Weights of decoder layer `layer` (1-based), nn.Linear layout [out, in], float32 arrays."""
    assert 1 <= layer <= shape.n_layers
    d, hq, hkv, dh, f = shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim
    dims = {"q": (hq * dh, d), "k": (hkv * dh, d), "v": (hkv * dh, d), "o": (d, hq * dh),
            "gate": (f, d), "up": (f, d), "down": (d, f)}
    # one generator per tensor: the draws are independent, so they run on a thread pool (numpy
    # fills arrays without holding the interpreter lock) with the same values as a serial loop
    with ThreadPoolExecutor(max_workers=min(len(dims), os.cpu_count() or 1)) as ex:
        drawn = list(ex.map(lambda n: _draw(shape, layer, _TENSOR_ID[n], dims[n]), dims))
    out = {"w_" + n: w for n, w in zip(dims, drawn)}
    out["g_attn"] = np.ones(d, np.float32)
    out["g_ffn"] = np.ones(d, np.float32)
    return out


def quantize_int8_rows(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 per output channel (row of an nn.Linear weight): s = max|w| / 127 and
    q = rint(w / s) (half to even) clamped to [-127, 127], in float32; an all-zero row gets
    s = 0 and q = 0.  Returns (q int8 [out, in], s float32 [out])."""
    w = np.asarray(w, np.float32)
    s = (np.abs(w).max(axis=1) / np.float32(127)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    q = np.clip(np.rint(w / safe[:, None]), -127, 127).astype(np.int8)
    return q, s


def layer_weights_int8(shape: ModelShape, layer: int) -> Dict[str, np.ndarray]:
    """Weights of decoder layer `layer` for the int8-weight run: the same float32 draws as
    layer_weights (before any bf16 rounding), each linear weight quantized per output row:
    q_<name> int8 [out, in] and s_<name> float32 [out]; norm gains are ones."""
    assert 1 <= layer <= shape.n_layers
    d, hq, hkv, dh, f = shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim
    dims = {"q": (hq * dh, d), "k": (hkv * dh, d), "v": (hkv * dh, d), "o": (d, hq * dh),
            "gate": (f, d), "up": (f, d), "down": (d, f)}

    def one(n):
        w = rng(_STREAM_WEIGHTS, layer, _TENSOR_ID[n]).standard_normal(dims[n], dtype=np.float32)
        w *= np.float32(0.02)
        return quantize_int8_rows(w)

    with ThreadPoolExecutor(max_workers=min(len(dims), os.cpu_count() or 1)) as ex:
        drawn = list(ex.map(one, dims))
    out = {}
    for n, (q, sc) in zip(dims, drawn):
        out["q_" + n] = q
        out["s_" + n] = sc
    out["g_attn"] = np.ones(d, np.float32)
    out["g_ffn"] = np.ones(d, np.float32)
    return out


def embedding(shape: ModelShape) -> np.ndarray:
    """Token embedding table [vocab, d] (float32 array; bf16-valued for bf16 shapes)."""
    return _draw(shape, 0, 0, (shape.vocab, shape.d_model))


def chunk_tokens(wl: Workload) -> List[np.ndarray]:
    return [rng(_STREAM_CHUNK, c).integers(0, wl.shape.vocab, n, dtype=np.int64).astype(np.int32)
            for c, n in enumerate(wl.chunk_lens)]


def query_tokens(wl: Workload) -> np.ndarray:
    return rng(_STREAM_QUERY).integers(0, wl.shape.vocab, wl.n_query, dtype=np.int64).astype(np.int32)


def all_tokens(wl: Workload) -> np.ndarray:
    return np.concatenate(chunk_tokens(wl) + [query_tokens(wl)]).astype(np.int32)


def chunk_offsets(wl: Workload) -> np.ndarray:
    """[n_chunks + 1] prefix offsets of the chunks in the fused sequence (last = context length)."""
    return np.concatenate([[0], np.cumsum(wl.chunk_lens)]).astype(np.int32)


def perturbation(layer: int, which: int, dims: Tuple[int, ...], scale: float) -> np.ndarray:
    """Seeded N(0, scale) noise (float32) used to give a literal layer-1 ranking a signal."""
    return (rng(_STREAM_PERTURB, layer, which).standard_normal(dims, dtype=np.float32)
            * np.float32(scale))


def kv_bytes_per_element(shape: ModelShape) -> int:
    return 4 if shape.dtype == "f32" else 2
