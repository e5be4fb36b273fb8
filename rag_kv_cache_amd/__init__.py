"""MI355X (gfx950) implementation of CacheBlend's per-layer KV fusion step.

The compute path is the HIP library librag_kv_cache_amd.so (C ABI in include/cacheblend.h);
`rag_kv_cache_amd._lib` binds it with ctypes and `rag_kv_cache_amd.pipeline` drives the layer
loop, using PyTorch only for device memory, pinned host memory and streams.
Build the library with `python -m rag_kv_cache_amd.build`.
"""
