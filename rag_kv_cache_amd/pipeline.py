"""Layer loop around the C ABI: weight upload, per-chunk cache build, blended prefill.

PyTorch is used here only to allocate device memory, pinned host memory and streams; every
step of the fusion runs in the HIP library through `rag_kv_cache_amd._lib`.

The flow follows the pages:
  * chunk caches: every chunk is prefilled alone at positions 0.. (CacheBlend explainer,
    background: each retrieved document's KV can be precomputed independently);
  * blended prefill: per layer, re-rotate the cache, recompute the selected rows, score and
    narrow them, scatter, attend, then the rest of the layer on the kept rows (CacheBlend
    review, per-layer flow; explainer, "Gradual filtering");
  * the cached KV either sits in HBM, or in pinned host memory and is fetched one layer
    ahead on a second stream (explainer, "Pipelined design": fetch_kv / synchronize).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
import torch

from . import _lib as L


def _ptr(t) -> int:
    """Address of a tensor, or an address given as an int (0 = NULL)."""
    if t is None:
        return 0
    return int(t) if isinstance(t, int) else int(t.data_ptr())


class Engine:
    """A library context plus the device weights of one model."""

    def __init__(self, shape, max_tokens: int, device: int = 0, copy_stream: bool = True,
                 streams: Optional[tuple] = None):
        """streams: optional (compute, copy) torch streams to use instead of new ones (e.g.
        torch.cuda.ExternalStream wrapping streams made elsewhere); copy may be None."""
        if not torch.cuda.is_available():
            raise RuntimeError("a ROCm GPU is required: the fusion step runs only in the HIP library")
        self.shape = shape
        self.device = torch.device("cuda", device)
        self.dtype = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        if streams is not None:
            self.compute, self.copy = streams
        else:
            self.compute = torch.cuda.Stream(self.device)
            self.copy = torch.cuda.Stream(self.device) if copy_stream else None
        desc = L.cb_model_desc(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads,
                               shape.head_dim, shape.ffn_dim, shape.vocab, max_tokens,
                               float(shape.rope_base), float(shape.rms_eps),
                               L.CB_BF16 if shape.dtype == "bf16" else L.CB_F32)
        self.max_tokens = max_tokens
        self.desc = desc
        self.ctx = L.cb_create(desc, device, self.compute.cuda_stream,
                               self.copy.cuda_stream if self.copy is not None else 0)
        self.weights: List[Dict[str, torch.Tensor]] = [None] * shape.n_layers
        self.emb: Optional[torch.Tensor] = None
        self._ws: Optional[torch.Tensor] = None

    def close(self):
        if self.ctx:
            L.cb_destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ weights
    def _dev(self, a: np.ndarray, dtype=None) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device).to(dtype or self.dtype)

    def load_layer(self, layer: int, w: Dict[str, np.ndarray]) -> None:
        """w: nn.Linear-layout float32 arrays w_q, w_k, w_v, w_o, w_gate, w_up, w_down, g_attn, g_ffn."""
        t = {
            "w_qkv": self._dev(np.concatenate([w["w_q"], w["w_k"], w["w_v"]])),
            "w_o": self._dev(w["w_o"]),
            "w_gate_up": self._dev(np.concatenate([w["w_gate"], w["w_up"]])),
            "w_down": self._dev(w["w_down"]),
            "g_attn": self._dev(w["g_attn"], torch.float32),
            "g_ffn": self._dev(w["g_ffn"], torch.float32),
        }
        self.weights[layer] = t
        L.cb_set_layer_weights(self.ctx, layer, _ptr(t["w_qkv"]), _ptr(t["w_o"]), _ptr(t["w_gate_up"]),
                               _ptr(t["w_down"]), _ptr(t["g_attn"]), _ptr(t["g_ffn"]))

    def load_layer_int8(self, layer: int, wq: Dict[str, np.ndarray]) -> None:
        """wq: int8 q_q, q_k, q_v, q_o, q_gate, q_up, q_down [out, in], their float32 per-row
        scales s_<name> [out], and the float32 gains g_attn, g_ffn (bf16 engines only)."""
        def dev8(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(self.device)

        def dev32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)

        t = {
            "w_qkv": dev8(np.concatenate([wq["q_q"], wq["q_k"], wq["q_v"]])),
            "w_o": dev8(wq["q_o"]),
            "w_gate_up": dev8(np.concatenate([wq["q_gate"], wq["q_up"]])),
            "w_down": dev8(wq["q_down"]),
            "s_qkv": dev32(np.concatenate([wq["s_q"], wq["s_k"], wq["s_v"]])),
            "s_o": dev32(wq["s_o"]),
            "s_gate_up": dev32(np.concatenate([wq["s_gate"], wq["s_up"]])),
            "s_down": dev32(wq["s_down"]),
            "g_attn": dev32(wq["g_attn"]),
            "g_ffn": dev32(wq["g_ffn"]),
        }
        self.weights[layer] = t
        L.cb_set_layer_weights_i8(self.ctx, layer, _ptr(t["w_qkv"]), _ptr(t["w_o"]), _ptr(t["w_gate_up"]),
                                  _ptr(t["w_down"]), _ptr(t["s_qkv"]), _ptr(t["s_o"]), _ptr(t["s_gate_up"]),
                                  _ptr(t["s_down"]), _ptr(t["g_attn"]), _ptr(t["g_ffn"]))

    def load_layer_device(self, layer: int, seed: int, int8: bool = False) -> None:
        """Random weights of `layer` drawn on the device: N(0, 0.02) float32 from torch's
        generator seeded with `seed`, then bf16 (or, with int8, quantized per output row: s =
        max|w| / 127, q = round half to even of w / s clamped to +-127); gains 1.  For benchmarks
        at sizes where drawing on the host would take minutes; the values differ from the
        fixtures' draws."""
        s = self.shape
        d, qd, kvd, f = s.d_model, s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim, s.ffn_dim
        g = torch.Generator(device=self.device)
        g.manual_seed(int(seed))

        def draw(rows, cols):
            w = torch.randn(rows, cols, generator=g, device=self.device, dtype=torch.float32)
            w.mul_(0.02)
            if not int8:
                return w.to(self.dtype), None
            sc = w.abs().amax(dim=1) / 127.0
            q = torch.round(w / torch.where(sc > 0, sc, torch.ones_like(sc))[:, None]).clamp_(-127, 127)
            return q.to(torch.int8), sc.contiguous()

        parts = {n: draw(r, c) for n, (r, c) in
                 {"qkv": (qd + 2 * kvd, d), "o": (d, qd), "gate_up": (2 * f, d), "down": (d, f)}.items()}
        t = {"w_" + n: parts[n][0] for n in parts}
        t["g_attn"] = torch.ones(d, dtype=torch.float32, device=self.device)
        t["g_ffn"] = torch.ones(d, dtype=torch.float32, device=self.device)
        self.weights[layer] = t
        if int8:
            for n in parts:
                t["s_" + n] = parts[n][1]
            L.cb_set_layer_weights_i8(self.ctx, layer, _ptr(t["w_qkv"]), _ptr(t["w_o"]), _ptr(t["w_gate_up"]),
                                      _ptr(t["w_down"]), _ptr(t["s_qkv"]), _ptr(t["s_o"]), _ptr(t["s_gate_up"]),
                                      _ptr(t["s_down"]), _ptr(t["g_attn"]), _ptr(t["g_ffn"]))
        else:
            L.cb_set_layer_weights(self.ctx, layer, _ptr(t["w_qkv"]), _ptr(t["w_o"]), _ptr(t["w_gate_up"]),
                                   _ptr(t["w_down"]), _ptr(t["g_attn"]), _ptr(t["g_ffn"]))

    def load_embedding_device(self, seed: int) -> None:
        """Embedding table [vocab, d] of N(0, 0.02) values drawn on the device (see load_layer_device)."""
        s = self.shape
        g = torch.Generator(device=self.device)
        g.manual_seed(int(seed))
        self.emb = (torch.randn(s.vocab, s.d_model, generator=g, device=self.device) * 0.02).to(self.dtype)

    def load_embedding(self, emb: np.ndarray) -> None:
        self.emb = self._dev(emb)

    def load_all(self, layer_weights: Callable[[int], Dict[str, np.ndarray]], emb: np.ndarray) -> None:
        """layer_weights(l) for l = 1..n_layers (1-based, as the fixtures number them)."""
        for l in range(self.shape.n_layers):
            self.load_layer(l, layer_weights(l + 1))
        self.load_embedding(emb)
        torch.cuda.synchronize(self.device)

    # ------------------------------------------------------------ buffers
    def workspace(self, n_tokens: int, n_sel_max: int) -> torch.Tensor:
        need = L.cb_workspace_size(self.ctx, n_tokens, n_sel_max)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def kv_empty(self, rows: int) -> torch.Tensor:
        s = self.shape
        return torch.zeros(rows, s.n_kv_heads, s.head_dim, dtype=self.dtype, device=self.device)

    # ------------------------------------------------------------ calls
    def embed(self, tokens: torch.Tensor, out: torch.Tensor) -> None:
        L.cb_embed(self.ctx, _ptr(tokens), int(tokens.numel()), _ptr(self.emb), _ptr(out))


@dataclass
class RunBuffers:
    """Device buffers of one blended prefill of up to n_tokens rows."""
    hidden: List[torch.Tensor]
    xnorm: List[torch.Tensor]     # normalized rows handed from one layer to the next
    sel: List[torch.Tensor]
    iota: torch.Tensor
    init_sel: torch.Tensor
    new_local: torch.Tensor
    out_sel: torch.Tensor
    dev: torch.Tensor
    tokens: torch.Tensor
    offsets: torch.Tensor
    ws: torch.Tensor


def make_buffers(eng: Engine, n_tokens: int, n_chunks: int) -> RunBuffers:
    s, dv = eng.shape, eng.device
    return RunBuffers(
        hidden=[torch.empty(n_tokens, s.d_model, dtype=torch.float32, device=dv) for _ in range(2)],
        xnorm=[torch.empty(n_tokens, s.d_model, dtype=eng.dtype, device=dv) for _ in range(2)],
        sel=[torch.empty(n_tokens, dtype=torch.int32, device=dv) for _ in range(2)],
        iota=torch.arange(n_tokens, dtype=torch.int32, device=dv),
        init_sel=torch.empty(n_tokens, dtype=torch.int32, device=dv),
        new_local=torch.empty(n_tokens, dtype=torch.int32, device=dv),
        out_sel=torch.empty(n_tokens, s.n_q_heads * s.head_dim, dtype=eng.dtype, device=dv),
        dev=torch.empty(n_tokens, dtype=torch.float32, device=dv),
        tokens=torch.empty(n_tokens, dtype=torch.int32, device=dv),
        offsets=torch.empty(n_chunks + 1, dtype=torch.int32, device=dv),
        ws=eng.workspace(n_tokens, n_tokens),
    )


@dataclass
class LayerRecord:
    sel: np.ndarray
    new_sel: np.ndarray
    deviation: Optional[np.ndarray]
    out_sel: Optional[np.ndarray]
    hidden_out: Optional[np.ndarray]
    h1: Optional[np.ndarray] = None    # residual after attention of the kept rows (fp32)
    act: Optional[np.ndarray] = None   # SwiGLU product of the kept rows (as float32)
    q: Optional[np.ndarray] = None     # Q of the kept rows after RoPE (as float32)


def workspace_q(eng: "Engine", ws: torch.Tensor, n_sel: int, n_new: int) -> np.ndarray:
    """Q of the kept rows (after RoPE) that cb_blend_layer(n_sel -> n_new rows) left in ws,
    as a host float32 array [n_new, H_q * d_h]; read it before cb_layer_rest reuses ws."""
    s = eng.shape
    v = L.cb_workspace_views(eng.ctx, n_sel, n_new == n_sel)
    es = 2 if eng.dtype == torch.bfloat16 else 4
    qd = s.n_q_heads * s.head_dim
    if n_new == 0:
        return np.zeros((0, qd), np.float32)
    rows = ws[v.q_offset: v.q_offset + ((n_new - 1) * v.q_ld + qd) * es].view(eng.dtype)
    return torch.as_strided(rows, (n_new, qd), (v.q_ld, 1)).float().cpu().numpy()


def workspace_intermediates(eng: "Engine", ws: torch.Tensor, n_sel: int, n_new: int):
    """h1 and the SwiGLU product that cb_layer_rest(n_sel -> n_new rows) left in ws, as host arrays."""
    s = eng.shape
    v = L.cb_workspace_views(eng.ctx, n_sel, n_new == n_sel)
    es = 2 if eng.dtype == torch.bfloat16 else 4
    h1 = ws[v.h1_offset: v.h1_offset + n_new * s.d_model * 4].view(torch.float32).reshape(n_new, s.d_model)
    act = ws[v.act_offset: v.act_offset + n_new * s.ffn_dim * es].view(eng.dtype).reshape(n_new, s.ffn_dim)
    return h1.cpu().numpy().copy(), act.float().cpu().numpy()


@dataclass
class RunResult:
    hidden: torch.Tensor          # [n_final, d] residual rows of the final kept set
    sel: torch.Tensor             # [n_final] their positions
    n_final: int
    records: List[LayerRecord] = field(default_factory=list)


def run_layers(eng: Engine, buf: RunBuffers, tokens: np.ndarray, offsets: Sequence[int], n_query: int,
               schedule: Sequence[float], fused: List[Sequence[torch.Tensor]],
               cache: Optional[List[Sequence[torch.Tensor]]] = None,
               host_cache: Optional[List[List[Sequence[torch.Tensor]]]] = None,
               record: bool = False, upload_inputs: bool = True,
               layer_events: Optional[list] = None, rotate_on_copy_stream: bool = False,
               initial_sel: Optional[Sequence[int]] = None, batch_rotation: bool = True,
               sel_uploaded: bool = False, paced: bool = False) -> RunResult:
    """Blended prefill over every layer.

    fused[l] = (K, V) device buffers [N, H_kv, d_h] of layer l (the fused cache, output).
    cache[l] = (K, V) device [N_ctx, H_kv, d_h] offset-0 chunk caches in prompt order (HBM
    mode: the position update copies them into fused[l] on the copy stream, two layers
    ahead); or host_cache[l][c] = (K, V) pinned host tensors of chunk c (prefetch mode:
    copied two layers ahead into fused[l] on the copy stream and updated in place there); or
    neither (the fused buffers are used as they are, e.g. a full prefill with no context).
    schedule[l] is the recompute ratio used at layer l.
    initial_sel: the rows recomputed at layer 1 (ascending, ending with every query row;
    default every row), e.g. the spatial seam-repair set of cb_seam_select, kept at every layer
    by a schedule of ratios >= 1.
    rotate_on_copy_stream (HBM mode): run the position update on the copy stream, two layers
    ahead (cb_fetch_layer_device), instead of inside cb_blend_layer on the compute stream.
    batch_rotation (HBM mode, otherwise): the position update of every layer in one launch
    before the first layer (cb_rotate_layers); False runs it inside each cb_blend_layer.
    upload_inputs=False reuses the token ids and offsets already on the device (a repeated
    step then enqueues no host-to-device copy); with initial_sel, sel_uploaded=True likewise
    reuses the rows and their token ids uploaded by an earlier call with the same initial_sel.
    record: True keeps every layer's sets, deviations, attention output, residual rows and
    intermediates on the host (the deviation is then written, which runs the deviation + scatter
    kernel at every layer); "sets" keeps only each layer's selected and kept positions, without
    changing which kernels run.
    paced (prefetch modes): layer l+2's fetch waits until the compute stream has reached layer l,
    so that the fetches spread over the step instead of running back to back at its start.  layer_events, if given, receives a CUDA event
    recorded on the compute stream before the first layer and after every layer.
    """
    s = eng.shape
    offs = [int(o) for o in offsets]
    n_chunks = len(offs) - 1
    n_ctx = offs[-1]
    n_tok = n_ctx + n_query
    assert len(tokens) == n_tok and len(schedule) == s.n_layers
    cs = eng.compute
    ctx = eng.ctx
    with torch.cuda.stream(cs):
        if initial_sel is not None:  # layer 1 embeds the selected rows only
            if not sel_uploaded:
                init = np.asarray(initial_sel, np.int32)
                buf.init_sel[: len(init)].copy_(torch.from_numpy(init), non_blocking=False)
                buf.tokens[: len(init)].copy_(torch.from_numpy(np.asarray(tokens, np.int32)[init]),
                                              non_blocking=False)
        elif upload_inputs:
            buf.tokens[:n_tok].copy_(torch.from_numpy(np.asarray(tokens, np.int32)), non_blocking=False)
        if upload_inputs or (initial_sel is not None and not sel_uploaded):
            buf.offsets[: n_chunks + 1].copy_(torch.tensor(offs, dtype=torch.int32))
    prefetch = host_cache is not None
    fetched = prefetch or (cache is not None and n_ctx > 0 and rotate_on_copy_stream)
    batched = cache is not None and not fetched and n_ctx > 0 and batch_rotation

    def fetch(l):
        # layer l's cache -> fused[l] with the position update, on the copy stream
        if l >= s.n_layers:
            return
        if prefetch:
            hk = [_ptr(host_cache[l][c][0]) for c in range(n_chunks)]
            hv = [_ptr(host_cache[l][c][1]) for c in range(n_chunks)]
            L.cb_fetch_layer(ctx, l, hk, hv, offs, n_chunks, _ptr(buf.offsets), _ptr(fused[l][0]), _ptr(fused[l][1]))
        elif fetched:
            L.cb_fetch_layer_device(ctx, l, _ptr(cache[l][0]), _ptr(cache[l][1]), offs, n_chunks, _ptr(buf.offsets),
                                    _ptr(fused[l][0]), _ptr(fused[l][1]))

    if fetched:
        fetch(0)
        fetch(1)
    def mark():
        if layer_events is not None:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(cs)
            layer_events.append(ev)

    if batched:  # every layer's position update in one launch on the compute stream
        L.cb_rotate_layers(ctx, 0, [_ptr(c[0]) for c in cache], [_ptr(c[1]) for c in cache], offs, n_chunks,
                           _ptr(buf.offsets), [_ptr(f[0]) for f in fused], [_ptr(f[1]) for f in fused])
    n_first = n_tok if initial_sel is None else len(initial_sel)
    L.cb_embed(ctx, _ptr(buf.tokens), n_first, _ptr(eng.emb), _ptr(buf.hidden[0]))
    mark()
    n_sel, cur = n_first, 0
    records = []
    ws = buf.ws
    for l in range(s.n_layers):
        if fetched:  # the fused buffer already holds the re-rotated cache
            L.cb_synchronize(ctx, l)
            if paced and l + 2 < s.n_layers:
                ev = torch.cuda.Event()
                ev.record(cs)
                eng.copy.wait_event(ev)
            fetch(l + 2)
            ck, cv = None, None
        elif cache is not None and not batched:  # position update inside cb_blend_layer (copy from the cache)
            ck, cv = cache[l]
        else:
            ck, cv = None, None
        fk, fv = fused[l]
        h_in, h_out = buf.hidden[cur], buf.hidden[1 - cur]
        sel_in = (buf.iota if initial_sel is None else buf.init_sel) if l == 0 else buf.sel[(l - 1) % 2]
        sel_out = buf.sel[l % 2]
        # layer l-1's cb_layer_rest already normalized this layer's input rows (x_sel)
        x_in = buf.xnorm[(l - 1) % 2] if l > 0 else None
        x_out = buf.xnorm[l % 2] if l + 1 < s.n_layers else None
        n_new = L.cb_blend_layer(ctx, l, _ptr(h_in), _ptr(ck), _ptr(cv), _ptr(fk), _ptr(fv),
                                 _ptr(buf.offsets) if n_chunks else 0, offs, n_chunks, _ptr(sel_in), n_sel,
                                 n_query, float(schedule[l]), _ptr(sel_out), _ptr(buf.new_local),
                                 _ptr(buf.out_sel), _ptr(buf.dev) if record is True else 0, _ptr(ws), ws.numel(),
                                 x_sel=_ptr(x_in))
        q_rec = None
        if record is True:
            cs.synchronize()
            q_rec = workspace_q(eng, ws, n_sel, n_new)
        L.cb_layer_rest(ctx, l, _ptr(h_in), n_sel, _ptr(buf.new_local), n_new, _ptr(buf.out_sel), _ptr(h_out),
                        _ptr(ws), ws.numel(), x_next=_ptr(x_out))
        if record == "sets":
            cs.synchronize()
            records.append(LayerRecord(sel=sel_in[:n_sel].cpu().numpy().copy(),
                                       new_sel=sel_out[:n_new].cpu().numpy().copy(),
                                       deviation=None, out_sel=None, hidden_out=None))
        elif record:
            cs.synchronize()
            h1, act = workspace_intermediates(eng, ws, n_sel, n_new)
            records.append(LayerRecord(
                sel=sel_in[:n_sel].cpu().numpy().copy(), new_sel=sel_out[:n_new].cpu().numpy().copy(),
                deviation=buf.dev[: n_sel - n_query].cpu().numpy().copy(),
                out_sel=buf.out_sel[:n_new].float().cpu().numpy().copy(),
                hidden_out=h_out[:n_new].cpu().numpy().copy(), h1=h1, act=act, q=q_rec))
        mark()
        n_sel, cur = n_new, 1 - cur
    final_sel = buf.sel[(s.n_layers - 1) % 2]
    return RunResult(hidden=buf.hidden[cur], sel=final_sel, n_final=n_sel, records=records)


def build_chunk_caches(eng: Engine, chunks: Sequence[np.ndarray], pinned_host: bool = False,
                       keep_device: bool = True):
    """Prefill every chunk alone at positions 0.. and keep its per-layer K/V.

    Returns (device_cache, host_cache): device_cache[l] = (K, V) [N_ctx, H_kv, d_h] with chunk c
    at rows [o_c, o_c + len_c) (or None); host_cache[l][c] = (K, V) pinned host tensors (or None).
    """
    s = eng.shape
    lens = [len(c) for c in chunks]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    n_ctx = int(offs[-1])
    dev_cache = [(eng.kv_empty(n_ctx), eng.kv_empty(n_ctx)) for _ in range(s.n_layers)] if keep_device else None
    host_cache = [[None] * len(chunks) for _ in range(s.n_layers)] if pinned_host else None
    lmax = max(lens)
    buf = make_buffers(eng, lmax, 0)
    tmp = [(eng.kv_empty(lmax), eng.kv_empty(lmax)) for _ in range(s.n_layers)]
    for c, toks in enumerate(chunks):
        n = len(toks)
        fused = [(k[:n], v[:n]) for k, v in tmp]
        run_layers(eng, buf, toks, [0], n, [1.0] * s.n_layers, fused)
        with torch.cuda.stream(eng.compute):
            for l in range(s.n_layers):
                if keep_device:
                    dev_cache[l][0][offs[c]:offs[c] + n].copy_(fused[l][0])
                    dev_cache[l][1][offs[c]:offs[c] + n].copy_(fused[l][1])
                if pinned_host:
                    hk = torch.empty(fused[l][0].shape, dtype=eng.dtype, pin_memory=True)
                    hv = torch.empty(fused[l][1].shape, dtype=eng.dtype, pin_memory=True)
                    hk.copy_(fused[l][0])
                    hv.copy_(fused[l][1])
                    host_cache[l][c] = (hk, hv)
        eng.compute.synchronize()
    return dev_cache, host_cache


class ChunkStore:
    """The library's host chunk store (cb_store_*) for one engine's model: per chunk, every
    layer's K and V of the chunk prefilled alone at positions 0.., found by its token ids."""

    def __init__(self, eng: Engine, max_chunk_tokens: int, n_slots: int, pinned: bool = True):
        self.n_layers = eng.shape.n_layers
        self.handle = L.cb_store_create(eng.desc, max_chunk_tokens, n_slots, pinned)

    def close(self):
        if self.handle:
            L.cb_store_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lookup(self, tokens, hold: bool = False) -> int:
        return L.cb_store_lookup(self.handle, tokens, None, hold)

    def release(self, slot: int) -> None:
        L.cb_store_release(self.handle, slot)

    def stats(self):
        return L.cb_store_get_stats(self.handle)

    def host_cache(self, slots: Sequence[int]) -> List[List[tuple]]:
        """host_cache[l][c] = (K address, V address) of layer l of the entry in slots[c], the
        form run_layers fetches from."""
        out = []
        for l in range(self.n_layers):
            out.append([L.cb_store_layer(self.handle, sl, l)[:2] for sl in slots])
        return out

    def lookup_prompt(self, chunks: Sequence[np.ndarray], hold: bool = True) -> Optional[List[int]]:
        """Slots of every chunk (each held when hold), or None, holding nothing, if any chunk
        is missing."""
        slots = []
        for c in chunks:
            sl = self.lookup(c, hold)
            if sl < 0:
                if hold:
                    for h in slots:
                        self.release(h)
                return None
            slots.append(sl)
        return slots


def produce_chunks(eng: Engine, store: ChunkStore, chunks: Sequence[np.ndarray], hold: bool = False) -> List[int]:
    """Chunk-cache producer: every chunk not yet in the store is prefilled alone at positions
    0.. (full recompute of every row at every layer) and each layer's K and V is copied from the
    device into its entry; entries become visible to lookups once the copies are done.
    Returns the slot of every chunk (held when hold; otherwise released before returning)."""
    s = eng.shape
    lmax = max(len(c) for c in chunks)
    buf = make_buffers(eng, lmax, 0)
    tmp = [(eng.kv_empty(lmax), eng.kv_empty(lmax)) for _ in range(s.n_layers)]
    slots, fresh, done = [], [], False
    try:
        for toks in chunks:
            slot, new, _ = L.cb_store_insert(store.handle, toks, None, True)
            slots.append(slot)
            if not new:
                continue
            n = len(toks)
            fused = [(k[:n], v[:n]) for k, v in tmp]
            run_layers(eng, buf, toks, [0], n, [1.0] * s.n_layers, fused)
            # same stream as the prefill: the next chunk's prefill reuses tmp only after these
            for l in range(s.n_layers):
                L.cb_store_put_layer(eng.ctx, store.handle, slot, l, _ptr(fused[l][0]), _ptr(fused[l][1]))
            fresh.append(slot)
        eng.compute.synchronize()
        for slot in fresh:
            L.cb_store_commit(store.handle, slot)
        done = True
    finally:
        if not hold or not done:
            for slot in slots:
                L.cb_store_release(store.handle, slot)
    return slots


def capture_step(eng: Engine, step: Callable[[], object]) -> "torch.cuda.CUDAGraph":
    """Record one call of `step` (a whole blended prefill enqueued on the compute stream) as a
    HIP graph; replaying it re-runs every kernel of the step with one launch.  The step must
    only enqueue library kernels on buffers that stay alive (no allocation, no host copy), and
    must have run once before so that one-time kernel attributes are set."""
    graph = torch.cuda.CUDAGraph()
    eng.compute.synchronize()
    with torch.cuda.graph(graph, stream=eng.compute):
        step()
    eng.compute.synchronize()
    return graph


def decode(eng: Engine, buf: RunBuffers, new_tokens: Sequence[int], n_past: int,
           fused: List[Sequence[torch.Tensor]]) -> torch.Tensor:
    """One decode step of len(new_tokens) tokens at positions n_past .. with the fused KV of
    every layer (rows 0 .. n_past - 1 filled by a blended prefill or earlier decode steps;
    the new rows are appended).  Returns the new rows' hidden state after the last layer
    ([n_new, d] fp32, a view into buf), enqueued on the engine's compute stream: synchronize
    it before reading.  Token ids are given: choosing them needs the LM head, which is not part
    of this library."""
    s = eng.shape
    n_new = len(new_tokens)
    cs = eng.compute
    ctx = eng.ctx
    with torch.cuda.stream(cs):
        buf.tokens[:n_new].copy_(torch.from_numpy(np.asarray(new_tokens, np.int32)), non_blocking=False)
        buf.init_sel[:n_new].copy_(torch.arange(n_past, n_past + n_new, dtype=torch.int32), non_blocking=False)
    L.cb_embed(ctx, _ptr(buf.tokens), n_new, _ptr(eng.emb), _ptr(buf.hidden[0]))
    ws = buf.ws
    cur = 0
    for l in range(s.n_layers):
        h_in, h_out = buf.hidden[cur], buf.hidden[1 - cur]
        # up to 4 rows go to the skinny products, which normalise the residual rows as they load
        # them; more rows take the normalised rows the previous layer's down-projection wrote
        x_in = buf.xnorm[(l - 1) % 2] if l > 0 and n_new > 4 else None
        x_out = buf.xnorm[l % 2] if l + 1 < s.n_layers and n_new > 4 else None
        L.cb_decode_layer(ctx, l, _ptr(h_in), _ptr(fused[l][0]), _ptr(fused[l][1]), n_past, n_new,
                          _ptr(buf.init_sel), _ptr(buf.out_sel), _ptr(ws), ws.numel(), x_new=_ptr(x_in))
        L.cb_layer_rest(ctx, l, _ptr(h_in), n_new, _ptr(buf.iota), n_new, _ptr(buf.out_sel), _ptr(h_out),
                        _ptr(ws), ws.numel(), x_next=_ptr(x_out))
        cur = 1 - cur
    return buf.hidden[cur][:n_new]
