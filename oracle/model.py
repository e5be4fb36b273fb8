"""Decoder-layer arithmetic of the oracle (float64 NumPy).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name the models (Mistral-7B, Yi-34B, Llama-70B; CacheBlend explainer,
"Experimental Results") but not their layer arithmetic.  The reading taken here
is the plain Llama-style pre-norm decoder those models share:
    h'  = h + Attn(RMSNorm(h)) W_o^T
    h'' = h' + W_down( silu(W_gate m) * (W_up m) ),  m = RMSNorm(h')
with RMSNorm eps 1e-6, no biases, contiguous GQA groups, and half-split RoPE
(pairs (i, i + d_h/2), angle p * base^(-2i/d_h)).

bf16 shapes: the GPU stores some intermediates in bfloat16.  `Precision.bf16`
rounds (to nearest, ties to even) at exactly those points so that values and
the top-k decision can be compared element by element:
  GEMM A operands (normalised rows, SwiGLU product), fresh K/V/Q after RoPE,
  the re-rotated cache, the attention output.
Everything else (accumulation, norms, softmax, residual stream, deviation)
stays in float64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of float64 data, via float32 bit patterns."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


@dataclass(frozen=True)
class Precision:
    """Where the path rounds.  kind 'f64': never (pure float64 semantics).
    kind 'bf16': round to bfloat16 at the storage points listed in the module doc."""
    kind: str = "f64"

    def store(self, x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float64)
        return round_bf16(x) if self.kind == "bf16" else x

    @staticmethod
    def for_dtype(dtype: str) -> "Precision":
        return Precision("bf16" if dtype == "bf16" else "f64")


F64 = Precision("f64")


# ---------------------------------------------------------------- RoPE
def rope_cos_sin(positions: Sequence[int], head_dim: int, base: float):
    """cos / sin of p * theta_i, theta_i = base^(-2i/d_h), i < d_h/2, in float64.  [n, d_h/2] each."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def rope_rotate(x: np.ndarray, positions: Sequence[int], base: float) -> np.ndarray:
    """Apply R(p) to every head of every row: x [n, H, d_h], positions [n].
    First half a, second half b of each head: (a, b) -> (a cos - b sin, b cos + a sin)."""
    x = np.asarray(x, dtype=np.float64)
    n, _, dh = x.shape
    c, s = rope_cos_sin(positions, dh, base)
    c, s = c[:, None, :], s[:, None, :]
    a, b = x[..., : dh // 2], x[..., dh // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_delta(k_cached: np.ndarray, chunk_offsets: Sequence[int], base: float) -> np.ndarray:
    """Position-encoding update of the CacheBlend explainer ("Position encoding update"):
    K_new[j] = R(dp_j) K_cached[j].  Every chunk was cached at offset 0, so dp_j is the
    chunk's offset o_c in the fused sequence for each of its rows (a reading: the
    workloads have no system prompt or separators).  k_cached [N_ctx, H_kv, d_h]."""
    offs = np.asarray(chunk_offsets)
    n_ctx = int(offs[-1])
    assert k_cached.shape[0] == n_ctx
    dp = np.empty(n_ctx, dtype=np.int64)
    for c in range(len(offs) - 1):
        dp[offs[c]:offs[c + 1]] = offs[c]
    return rope_rotate(k_cached, dp, base)


# ---------------------------------------------------------------- layer pieces
def rmsnorm(h: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * np.asarray(gain, np.float64)


def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [n, in] times nn.Linear weight w [out, in] -> [n, out] (float64 accumulation)."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: Sequence[int]) -> np.ndarray:
    """Causal GQA attention for an arbitrary set of query rows (CacheBlend review: the
    selected tokens' queries attend, under the causal mask, to all available K/V).
    q [n, H_q, d_h] with absolute positions q_pos [n]; k, v [N, H_kv, d_h] indexed by position.
    Query row i sees keys 0..q_pos[i] (diagonal included); scale 1/sqrt(d_h);
    query head h reads KV head h // (H_q / H_kv)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, hq, dh = q.shape
    nk, hkv, _ = k.shape
    group = hq // hkv
    q_pos = np.asarray(q_pos, dtype=np.int64)
    assert n == 0 or q_pos.max() < nk
    out = np.zeros((n, hq, dh))
    if n == 0:
        return out
    keys = int(q_pos.max()) + 1
    masked = np.arange(keys)[None, :] > q_pos[:, None]
    for h in range(hq):
        g = h // group
        s = (q[:, h, :] @ k[:keys, g, :].T) / np.sqrt(dh)
        s[masked] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:keys, g, :]
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def swiglu(h1: np.ndarray, w: Dict[str, np.ndarray], eps: float, prec: Precision) -> np.ndarray:
    """The FFN's inner activations: silu(W_gate m) * W_up m with m = RMSNorm(h1) (stored)."""
    m = prec.store(rmsnorm(h1, w["g_ffn"], eps))
    return prec.store(silu(project(m, w["w_gate"])) * project(m, w["w_up"]))


def mlp(h1: np.ndarray, w: Dict[str, np.ndarray], eps: float, prec: Precision, act=None) -> np.ndarray:
    """Second half of the layer: h1 + W_down(silu(W_gate m) * W_up m), m = RMSNorm(h1).
    act: the inner activations if already known (swiglu of the same h1), else computed."""
    if act is None:
        act = swiglu(h1, w, eps, prec)
    return np.asarray(h1, np.float64) + project(act, w["w_down"])


# ---------------------------------------------------------------- full prefill (ground truth)
def dequantize(wq: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """The int8-weight model as the oracle runs it: every linear weight is q * s in float32
    (q int8 [out, in], s float32 per output row), the norm gains as given.  Reading (no page
    fixes a weight format): symmetric per-output-channel int8 of the same float32 draws."""
    out = {"g_attn": np.asarray(wq["g_attn"], np.float32), "g_ffn": np.asarray(wq["g_ffn"], np.float32)}
    for n in ("q", "k", "v", "o", "gate", "up", "down"):
        out["w_" + n] = np.asarray(wq["q_" + n], np.float32) * np.asarray(wq["s_" + n], np.float32)[:, None]
    return out


def full_prefill(shape, weights: List[Dict[str, np.ndarray]], emb: np.ndarray, tokens: np.ndarray,
                 prec: Precision = F64, start_pos: int = 0):
    """Ordinary prefill of `tokens` at positions start_pos.. (every row, every layer).
    Returns dict(k=[L][N,H_kv,d_h], v=[...], hidden=[L+1][N,d] residual streams)."""
    hq, hkv, dh = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    n = len(tokens)
    pos = np.arange(start_pos, start_pos + n)
    h = np.asarray(emb[np.asarray(tokens)], np.float64)
    ks, vs, hs = [], [], [h]
    for w in weights:
        x = prec.store(rmsnorm(h, w["g_attn"], shape.rms_eps))
        q = prec.store(rope_rotate(project(x, w["w_q"]).reshape(n, hq, dh), pos, shape.rope_base))
        k = prec.store(rope_rotate(project(x, w["w_k"]).reshape(n, hkv, dh), pos, shape.rope_base))
        v = prec.store(project(x, w["w_v"]).reshape(n, hkv, dh))
        # keys are indexed by absolute position; pad the first start_pos slots (never attended)
        kk = np.concatenate([np.zeros((start_pos, hkv, dh)), k]) if start_pos else k
        vv = np.concatenate([np.zeros((start_pos, hkv, dh)), v]) if start_pos else v
        att = prec.store(causal_attention(q, kk, vv, pos)).reshape(n, hq * dh)
        h1 = h + project(att, w["w_o"])
        h = mlp(h1, w, shape.rms_eps, prec)
        ks.append(k)
        vs.append(v)
        hs.append(h)
    return {"k": ks, "v": vs, "hidden": hs}


def chunk_caches(shape, weights, emb, chunks: Sequence[np.ndarray], prec: Precision = F64):
    """Per-chunk KV caches: each chunk prefilled alone at positions 0.. (the pages' premise:
    every retrieved chunk's KV is precomputed independently).  Returns [chunk][layer] (k, v)."""
    out = []
    for toks in chunks:
        r = full_prefill(shape, weights, emb, toks, prec)
        out.append(list(zip(r["k"], r["v"])))
    return out


def cache_nbytes(shape, n_tokens: int, elem_bytes: int) -> int:
    """Bytes of a KV cache holding n_tokens over all layers: one K and one V row of
    H_kv * d_h elements per token per layer (LMCache blog, part 1 formula)."""
    return 2 * shape.n_layers * shape.n_kv_heads * shape.head_dim * elem_bytes * n_tokens
