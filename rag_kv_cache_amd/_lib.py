"""ctypes binding of include/cacheblend.h: the same names, argument marshalling only.

Device pointers are passed as Python ints (0 = NULL); host arrays as sequences of ints.
Every function raises CbError when the library returns a non-OK status.  There is no
fallback: if the HIP library is not built, importing this module fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librag_kv_cache_amd.so")

CB_OK, CB_EINVAL, CB_ESHAPE, CB_ESTATE, CB_EHIP, CB_ENOMEM, CB_EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "CB_OK", -1: "CB_EINVAL", -2: "CB_ESHAPE", -3: "CB_ESTATE", -4: "CB_EHIP",
                -5: "CB_ENOMEM", -6: "CB_EUNSUPPORTED"}
CB_F32, CB_BF16 = 0, 1
(CB_K_EMBED, CB_K_ROPE, CB_K_RMSNORM, CB_K_GEMM_KV, CB_K_DEV_SCATTER, CB_K_TOPK, CB_K_GEMM_Q, CB_K_ATTN,
 CB_K_GEMM_O, CB_K_GEMM_GATE_UP, CB_K_GEMM_DOWN, CB_K_FETCH, CB_K_COUNT) = range(13)
KERNEL_NAMES = ["embed", "rope_delta", "rmsnorm", "gemm_kv", "dev_scatter", "topk", "gemm_q", "attention",
                "gemm_o", "gemm_gate_up", "gemm_down", "fetch"]


class CbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class cb_model_desc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab_size", C.c_int32), ("max_tokens", C.c_int32), ("rope_base", C.c_float),
                ("rms_eps", C.c_float), ("dtype", C.c_int32)]


class cb_layer_weights(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("w_gate_up", C.c_void_p),
                ("w_down", C.c_void_p), ("g_attn", C.c_void_p), ("g_ffn", C.c_void_p)]


class cb_layer_weights_i8(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("w_gate_up", C.c_void_p), ("w_down", C.c_void_p),
                ("s_qkv", C.c_void_p), ("s_o", C.c_void_p), ("s_gate_up", C.c_void_p), ("s_down", C.c_void_p),
                ("g_attn", C.c_void_p), ("g_ffn", C.c_void_p)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library {LIB_PATH} is not built; run `python -m rag_kv_cache_amd.build`")
    return C.CDLL(LIB_PATH)


_L = _load()
_P = C.c_void_p
_I = C.c_int32
_L.cb_last_error.restype = C.c_char_p
_L.cb_last_error.argtypes = []
_SIGS = {
    "cb_create": [C.POINTER(cb_model_desc), _I, _P, _P, C.POINTER(_P)],
    "cb_destroy": [_P],
    "cb_set_layer_weights": [_P, _I, C.POINTER(cb_layer_weights)],
    "cb_set_layer_weights_i8": [_P, _I, C.POINTER(cb_layer_weights_i8)],
    "cb_workspace_size": [_P, _I, _I, C.POINTER(C.c_size_t)],
    "cb_embed": [_P, _P, _I, _P, _P],
    "cb_fetch_layer": [_P, _I, C.POINTER(_P), C.POINTER(_P), C.POINTER(_I), _I, _P, _P, _P],
    "cb_fetch_layer_device": [_P, _I, _P, _P, C.POINTER(_I), _I, _P, _P, _P],
    "cb_set_fetch_mode": [_P, _I],
    "cb_set_fetch_launch": [_P, _I, _I, _I],
    "cb_rotate_layers": [_P, _I, _I, C.POINTER(_P), C.POINTER(_P), C.POINTER(_I), _I, _P, C.POINTER(_P), C.POINTER(_P)],
    "cb_synchronize": [_P, _I],
    "cb_blend_layer": [_P, _I, _P, _P, _P, _P, _P, _P, _P, C.POINTER(_I), _I, _P, _I, _I, C.c_float, _P, _P,
                       C.POINTER(_I), _P, _P, _P, C.c_size_t],
    "cb_layer_rest": [_P, _I, _P, _I, _P, _I, _P, _P, _P, _P, C.c_size_t],
    "cb_blend_layer_static": [_P, _I, _P, _P, _P, _P, _P, _P, _P, C.POINTER(_I), _I, _P, _I, _I, C.c_float, _P,
                              _P, C.POINTER(_I), _P, _P],
    "cb_decode_layer": [_P, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P, C.c_size_t],
    "cb_workspace_views": [_P, _I, _I, _P],
    "cb_set_score_mode": [_P, _I],
    "cb_seam_select": [C.POINTER(_I), _I, _I, _I, C.POINTER(_I), _I, C.POINTER(_I)],
    "cb_plan_ratio": [_I, _I, C.c_double, C.c_double, C.c_double, C.c_double, C.c_float, C.c_float, _P],
    "cb_plan_ratio_measured": [_I, C.c_double, C.c_double, C.c_double, C.c_double, C.c_double, C.c_double,
                               C.c_double, C.c_double, C.c_float, C.c_float, _P],
    "cb_sha256": [_P, C.c_size_t, _P],
    "cb_chunk_key": [_P, _I, _P, _I, C.POINTER(C.c_uint64)],
    "cb_store_create": [C.POINTER(cb_model_desc), _I, _I, _I, C.POINTER(_P)],
    "cb_store_destroy": [_P],
    "cb_store_lookup": [_P, _P, _I, _P, _I, _I, C.POINTER(_I)],
    "cb_store_insert": [_P, _P, _I, _P, _I, _I, C.POINTER(_I), C.POINTER(_I), C.POINTER(_I)],
    "cb_store_commit": [_P, _I],
    "cb_store_release": [_P, _I],
    "cb_store_layer": [_P, _I, _I, C.POINTER(_P), C.POINTER(_P), C.POINTER(_I)],
    "cb_store_put_layer": [_P, _P, _I, _I, _P, _P],
    "cb_store_get_stats": [_P, _P],
    "cb_profile_enable": [_P, _I],
    "cb_profile_read": [_P, _I, C.POINTER(C.c_double), C.POINTER(C.c_int64), C.POINTER(C.c_double)],
}
for _name, _args in _SIGS.items():
    _f = getattr(_L, _name)
    _f.argtypes = _args
    _f.restype = C.c_int


def _check(status: int) -> None:
    if status != CB_OK:
        raise CbError(status, _L.cb_last_error().decode())


def _i32(seq: Sequence[int]):
    return (_I * len(seq))(*[int(v) for v in seq])


def cb_last_error() -> str:
    return _L.cb_last_error().decode()


def cb_create(desc: cb_model_desc, device: int = 0, compute_stream: int = 0, copy_stream: int = 0) -> int:
    out = _P()
    _check(_L.cb_create(C.byref(desc), device, compute_stream or None, copy_stream or None, C.byref(out)))
    return out.value


def cb_destroy(ctx: int) -> None:
    _check(_L.cb_destroy(ctx))


def cb_set_layer_weights(ctx: int, layer: int, w_qkv: int, w_o: int, w_gate_up: int, w_down: int,
                         g_attn: int, g_ffn: int) -> None:
    w = cb_layer_weights(w_qkv, w_o, w_gate_up, w_down, g_attn, g_ffn)
    _check(_L.cb_set_layer_weights(ctx, layer, C.byref(w)))


def cb_set_layer_weights_i8(ctx: int, layer: int, w_qkv: int, w_o: int, w_gate_up: int, w_down: int,
                            s_qkv: int, s_o: int, s_gate_up: int, s_down: int, g_attn: int, g_ffn: int) -> None:
    w = cb_layer_weights_i8(w_qkv, w_o, w_gate_up, w_down, s_qkv, s_o, s_gate_up, s_down, g_attn, g_ffn)
    _check(_L.cb_set_layer_weights_i8(ctx, layer, C.byref(w)))


def cb_workspace_size(ctx: int, n_tokens: int, n_sel_max: int) -> int:
    out = C.c_size_t()
    _check(_L.cb_workspace_size(ctx, n_tokens, n_sel_max, C.byref(out)))
    return out.value


def cb_embed(ctx: int, tokens: int, n: int, table: int, hidden_out: int) -> None:
    _check(_L.cb_embed(ctx, tokens, n, table, hidden_out))


def cb_fetch_layer(ctx: int, layer: int, host_k: Sequence[int], host_v: Sequence[int],
                   chunk_offsets_host: Sequence[int], n_chunks: int, chunk_offsets_dev: int, fused_k: int,
                   fused_v: int) -> None:
    hk = (_P * max(len(host_k), 1))(*host_k)
    hv = (_P * max(len(host_v), 1))(*host_v)
    _check(_L.cb_fetch_layer(ctx, layer, hk, hv, _i32(chunk_offsets_host), n_chunks, chunk_offsets_dev or None,
                             fused_k, fused_v))


def cb_fetch_layer_device(ctx: int, layer: int, cache_k: int, cache_v: int, chunk_offsets_host: Sequence[int],
                          n_chunks: int, chunk_offsets_dev: int, fused_k: int, fused_v: int) -> None:
    _check(_L.cb_fetch_layer_device(ctx, layer, cache_k or None, cache_v or None, _i32(chunk_offsets_host),
                                    n_chunks, chunk_offsets_dev or None, fused_k, fused_v))


CB_FETCH_COPY, CB_FETCH_KERNEL, CB_FETCH_AUTO = 0, 1, 2


def cb_set_fetch_mode(ctx: int, mode: int) -> None:
    _check(_L.cb_set_fetch_mode(ctx, mode))


def cb_set_fetch_launch(ctx: int, blocks: int, threads: int, unroll: int) -> None:
    _check(_L.cb_set_fetch_launch(ctx, blocks, threads, unroll))


def cb_rotate_layers(ctx: int, first_layer: int, cache_k: Sequence[int], cache_v: Sequence[int],
                     chunk_offsets: Sequence[int], n_chunks: int, chunk_offsets_dev: int, fused_k: Sequence[int],
                     fused_v: Sequence[int]) -> None:
    n = len(cache_k)
    assert len(cache_v) == len(fused_k) == len(fused_v) == n
    arr = lambda v: (_P * max(n, 1))(*[int(x) or None for x in v])
    _check(_L.cb_rotate_layers(ctx, first_layer, n, arr(cache_k), arr(cache_v), _i32(chunk_offsets), n_chunks,
                               chunk_offsets_dev or None, arr(fused_k), arr(fused_v)))


def cb_synchronize(ctx: int, layer: int) -> None:
    _check(_L.cb_synchronize(ctx, layer))


def cb_blend_layer(ctx: int, layer: int, hidden_sel: int, kv_cached_k: int, kv_cached_v: int,
                   kv_fused_k: int, kv_fused_v: int, chunk_offsets_dev: int,
                   chunk_offsets_host: Sequence[int], n_chunks: int, sel_idx: int, n_sel: int,
                   n_query: int, ratio: float, new_sel_idx: int, new_sel_local: int, out_sel: int,
                   deviation: int, workspace: int, workspace_bytes: int, x_sel: int = 0) -> int:
    """Returns n_new (= k + n_query)."""
    n_new = _I()
    _check(_L.cb_blend_layer(ctx, layer, hidden_sel, x_sel or None, kv_cached_k or None, kv_cached_v or None, kv_fused_k,
                             kv_fused_v, chunk_offsets_dev or None, _i32(chunk_offsets_host), n_chunks,
                             sel_idx, n_sel, n_query, ratio, new_sel_idx, new_sel_local, C.byref(n_new),
                             out_sel, deviation or None, workspace, workspace_bytes))
    return n_new.value


def cb_blend_layer_static(ctx: int, layer: int, hidden_sel: int, kv_cached_k: int, kv_cached_v: int,
                          kv_fused_k: int, kv_fused_v: int, chunk_offsets_dev: int,
                          chunk_offsets_host: Sequence[int], n_chunks: int, sel_idx: int, n_sel: int,
                          n_query: int, ratio: float, new_sel_idx: int, new_sel_local: int, out_sel: int,
                          deviation: int, x_sel: int = 0) -> int:
    """cb_blend_layer on the library's static workspace (no workspace argument).  Returns n_new."""
    n_new = _I()
    _check(_L.cb_blend_layer_static(ctx, layer, hidden_sel, x_sel or None, kv_cached_k or None, kv_cached_v or None,
                                    kv_fused_k, kv_fused_v, chunk_offsets_dev or None, _i32(chunk_offsets_host),
                                    n_chunks, sel_idx, n_sel, n_query, ratio, new_sel_idx, new_sel_local,
                                    C.byref(n_new), out_sel, deviation or None))
    return n_new.value


def cb_decode_layer(ctx: int, layer: int, hidden_new: int, kv_fused_k: int, kv_fused_v: int, n_past: int,
                    n_new: int, pos_dev: int, out_sel: int, workspace: int, workspace_bytes: int,
                    x_new: int = 0) -> None:
    _check(_L.cb_decode_layer(ctx, layer, hidden_new, x_new or None, kv_fused_k, kv_fused_v, n_past, n_new,
                              pos_dev, out_sel, workspace, workspace_bytes))


def cb_layer_rest(ctx: int, layer: int, hidden_sel: int, n_sel: int, new_sel_local: int, n_new: int,
                  out_sel: int, hidden_next: int, workspace: int, workspace_bytes: int, x_next: int = 0) -> None:
    _check(_L.cb_layer_rest(ctx, layer, hidden_sel, n_sel, new_sel_local, n_new, out_sel, hidden_next,
                            x_next or None, workspace, workspace_bytes))


class cb_ws_views(C.Structure):
    _fields_ = [("q_offset", C.c_size_t), ("q_ld", C.c_int32), ("h1_offset", C.c_size_t),
                ("act_offset", C.c_size_t)]


def cb_workspace_views(ctx: int, n_sel: int, all_kept: bool) -> "cb_ws_views":
    """Byte offsets (and Q's row stride) of the intermediates the calls leave in the workspace."""
    out = cb_ws_views()
    _check(_L.cb_workspace_views(ctx, n_sel, int(bool(all_kept)), C.byref(out)))
    return out


CB_SCORE_L2, CB_SCORE_COSINE = 0, 1


def cb_set_score_mode(ctx: int, mode: int) -> None:
    _check(_L.cb_set_score_mode(ctx, mode))


def cb_seam_select(chunk_offsets_host: Sequence[int], n_chunks: int, n_query: int, window: int):
    """The spatial seam-repair set (positions before every chunk boundary, then the query rows)."""
    n = _I()
    _L.cb_seam_select(_i32(chunk_offsets_host), n_chunks, n_query, window, None, 0, C.byref(n))
    out = (_I * max(n.value, 1))()
    _check(_L.cb_seam_select(_i32(chunk_offsets_host), n_chunks, n_query, window, out, n.value, C.byref(n)))
    return [out[i] for i in range(n.value)]


class cb_ratio_plan(C.Structure):
    _fields_ = [("load", _I), ("ratio", C.c_float), ("t_load_layer", C.c_double), ("t_recompute_layer", C.c_double),
                ("t_layer", C.c_double), ("t_total", C.c_double), ("break_even_bandwidth", C.c_double)]


def cb_plan_ratio(n_ctx: int, n_layers: int, kv_bytes_per_token_layer: float, bandwidth: float,
                  prefill_s_per_token: float, latency_layer_s: float, r_min: float, r_max: float) -> cb_ratio_plan:
    out = cb_ratio_plan()
    _check(_L.cb_plan_ratio(n_ctx, n_layers, kv_bytes_per_token_layer, bandwidth, prefill_s_per_token,
                            latency_layer_s, r_min, r_max, C.byref(out)))
    return out


def cb_plan_ratio_measured(n_layers: int, kv_bytes_layer: float, bandwidth: float, latency_layer_s: float,
                           t_first_layer: float, t_full_layer: float, t_fixed_layer: float, r_min: float,
                           r_max: float, t_select_layer: float = 0.0, contention: float = 0.0) -> cb_ratio_plan:
    out = cb_ratio_plan()
    _check(_L.cb_plan_ratio_measured(n_layers, kv_bytes_layer, bandwidth, latency_layer_s, t_first_layer,
                                     t_select_layer, t_full_layer, t_fixed_layer, contention, r_min, r_max,
                                     C.byref(out)))
    return out


def _arr(a, dtype):
    """(keep-alive array, address) of a contiguous host copy, or (None, 0) when empty."""
    a = np.ascontiguousarray(np.asarray(a if a is not None else [], dtype=dtype))
    return a, (a.ctypes.data if a.size else 0)


def cb_sha256(data: bytes) -> bytes:
    out = (C.c_uint8 * 32)()
    buf = C.create_string_buffer(bytes(data), len(data)) if data else None
    _check(_L.cb_sha256(C.addressof(buf) if buf is not None else None, len(data), C.addressof(out)))
    return bytes(out)


def cb_chunk_key(tokens, prior=None) -> int:
    t, tp = _arr(tokens, np.int32)
    p, pp = _arr(prior, np.uint64)
    k = C.c_uint64()
    _check(_L.cb_chunk_key(tp or None, t.size, pp or None, p.size, C.byref(k)))
    return k.value


class cb_store_stats(C.Structure):
    _fields_ = [("hits", C.c_int64), ("misses", C.c_int64), ("evictions", C.c_int64), ("entries", _I),
                ("capacity", _I), ("index_bytes", C.c_size_t), ("arena_bytes", C.c_size_t),
                ("slot_bytes", C.c_size_t)]


def cb_store_create(desc: cb_model_desc, max_chunk_tokens: int, n_slots: int, pinned: bool) -> int:
    out = _P()
    _check(_L.cb_store_create(C.byref(desc), max_chunk_tokens, n_slots, 1 if pinned else 0, C.byref(out)))
    return out.value


def cb_store_destroy(store: int) -> None:
    _check(_L.cb_store_destroy(store))


def cb_store_lookup(store: int, tokens, prior=None, pin: bool = False) -> int:
    t, tp = _arr(tokens, np.int32)
    p, pp = _arr(prior, np.uint64)
    slot = _I()
    _check(_L.cb_store_lookup(store, tp or None, t.size, pp or None, p.size, 1 if pin else 0, C.byref(slot)))
    return slot.value


def cb_store_insert(store: int, tokens, prior=None, pin: bool = False):
    """Returns (slot, is_new, evicted_slot or -1)."""
    t, tp = _arr(tokens, np.int32)
    p, pp = _arr(prior, np.uint64)
    slot, new, ev = _I(), _I(), _I()
    _check(_L.cb_store_insert(store, tp or None, t.size, pp or None, p.size, 1 if pin else 0, C.byref(slot),
                              C.byref(new), C.byref(ev)))
    return slot.value, bool(new.value), ev.value


def cb_store_commit(store: int, slot: int) -> None:
    _check(_L.cb_store_commit(store, slot))


def cb_store_release(store: int, slot: int) -> None:
    _check(_L.cb_store_release(store, slot))


def cb_store_layer(store: int, slot: int, layer: int):
    """Returns (host K address, host V address, n_tokens)."""
    k, v, n = _P(), _P(), _I()
    _check(_L.cb_store_layer(store, slot, layer, C.byref(k), C.byref(v), C.byref(n)))
    return k.value, v.value, n.value


def cb_store_put_layer(ctx: int, store: int, slot: int, layer: int, dev_k: int, dev_v: int) -> None:
    _check(_L.cb_store_put_layer(ctx, store, slot, layer, dev_k, dev_v))


def cb_store_get_stats(store: int) -> cb_store_stats:
    out = cb_store_stats()
    _check(_L.cb_store_get_stats(store, C.byref(out)))
    return out


def cb_profile_enable(ctx: int, on: bool) -> None:
    _check(_L.cb_profile_enable(ctx, 1 if on else 0))


def cb_profile_read(ctx: int, kernel_id: int):
    ms, n, work = C.c_double(), C.c_int64(), C.c_double()
    _check(_L.cb_profile_read(ctx, kernel_id, C.byref(ms), C.byref(n), C.byref(work)))
    return ms.value, n.value, work.value


def exported_symbols() -> list:
    return [n for n in list(_SIGS) + ["cb_last_error"] if hasattr(_L, n)]
