"""CPU oracle for CacheBlend's per-layer KV fusion step (selective KV recompute).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check in
__graft_entry__ and the benchmark's CPU-baseline leg may import or run anything
in this package.  The HIP library never calls it and shares no code with it.

Everything here is plain NumPy in float64, written step by step from the pages:

* CacheBlend explainer (0h-n0.github.io), sections "HKVD token selection"
  (the KV deviation equation), "Gradual filtering", "Position encoding update"
  (K_new = R(dp) K_cached) and "Pipelined design" (T_recompute / T_load);
* the CacheBlend review (jaehun.me), section on the per-layer flow of the
  selected tokens (fresh Q/K/V for selected rows, cached K/V for the rest,
  selected queries attend causally to all available K/V, output to the next
  layer).

Where the pages are silent the oracle takes the plainest reading; each such
reading is named in the function that takes it.

Parity status per function (what pins each one, see tests/test_oracle_*.py):
  rope_* ............ closed-form rotation algebra, complex-multiplication identity
  rmsnorm, project,
  attention, mlp .... Hugging Face Llama forward in float32 (library routine),
                      torch scaled_dot_product_attention on CPU, brute-force softmax
  topk_select ....... exhaustive brute force with forced ties
  blend_layer,
  blended_prefill ... special cases: ratio 1 = full prefill, single chunk at
                      offset 0 = exact cache, ratio 0 + single chunk = cache,
                      layer-1 identity, chunk-0 zero deviation, set invariants
  cosine_deviation .. identical / opposite / orthogonal rows, scale invariance, the
                      closed form 1 - cos(theta) for a rotation by theta
  seam_positions .... hand-worked boundary windows (short chunks, window > chunk)
  decode_step ....... after a full-recompute prefill, decoding equals full prefill of the
                      longer prompt; one step of two tokens equals two steps of one
  controller ........ the break-even and load/recompute numbers the LMCache page and the
                      CacheBlend review print
  store ............. FIPS 180-2 SHA-256 examples rebuilt from token and key bytes, the
                      LRU cyclic-scan trap the LMCache page measures, LRU's stack property,
                      a hand-worked eviction sequence
  dequantize ........ q * s per output row in float32 against hand-worked rows
  which rows are HKVD on random weights ... parity unpinned (the pages print no
                      worked example; only the invariants above constrain it)
"""
from .model import (  # noqa: F401
    Precision, F64, round_bf16, rope_cos_sin, rope_rotate, rope_delta, rmsnorm, project,
    causal_attention, swiglu, mlp, full_prefill, chunk_caches, cache_nbytes, dequantize,
)
from .blend import (  # noqa: F401
    k_for_ratio, topk_select, kv_deviation, cosine_deviation, seam_positions, blend_layer,
    attn_residual, layer_rest, fuse_cache, blended_prefill, decode_step,
)
from . import controller, store  # noqa: F401
