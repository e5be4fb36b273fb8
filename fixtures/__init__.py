"""Seeded synthetic inputs shared by the oracle, the GPU tests and the benchmark.

This package holds data only: model shapes, workload layouts, seeded weight and
token draws.  It contains none of the fusion method's arithmetic, so that the
CPU oracle and the HIP path stay independent of each other.
"""
from .synth import (  # noqa: F401
    SEED, ModelShape, Workload, CONFIGS, get_config, rng, layer_weights, embedding,
    chunk_tokens, query_tokens, all_tokens, chunk_offsets, perturbation, to_bf16_values,
    to_bf16_bits, kv_bytes_per_element, quantize_int8_rows, layer_weights_int8,
)
