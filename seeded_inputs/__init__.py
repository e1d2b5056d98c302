"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This package defines the *data* of every workload: model shapes, the random-init
weights (bf16 or int4 codes + bf16 scales), prompt ids and draft windows.  It
holds none of the forward pass's arithmetic (no norms, attention, GEMMs or
argmax); both the oracle and the GPU path consume what it produces.
"""
from .configs import ModelConfig, PRESETS, get_config, layer_variant  # noqa: F401
from .weights import (  # noqa: F401
    bf16_bits_from_f32, f32_from_bf16_bits, generate_weights, quantize_int4_g64,
    ModelWeights,
)
from .tokens import prompt_ids, draft_window, DraftSource, PATTERNS  # noqa: F401
