"""Seeded synthetic inputs (shapes, weights, cache prefill, tokens).

Both the GPU path's tests and the CPU oracle draw their inputs from here; the
module holds input recipes and storage encodings only.
"""
from .configs import CONFIGS, DecodeConfig, tiny, token_bytes, head_bytes, layer_weight_bytes, kv_bytes, elem_bytes  # noqa: F401
from .gen import (Stored, layer_weights, prefill, model_globals, embedding, tokens, f32_to_bf16_bits,  # noqa: F401
                  rand_f32, rand_matrix, rand_norm, rand_cache)
