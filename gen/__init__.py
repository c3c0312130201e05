"""Seeded synthetic inputs for the MoE expert layer.

This package produces inputs only: bf16 token activations, fp32 router logits,
quantized expert weights laid out as VRAM slots, and the slot table. It holds
none of the layer's own arithmetic (routing weights, align, FFN, combine); the
HIP path and the CPU oracle both consume what it produces and nothing else is
shared between them.
"""
from .configs import CONFIGS, Config, config_by_name  # noqa: F401
from .inputs import (  # noqa: F401
    FMT_FP8_E4M3_ROW, FMT_INT4_G128, slot_layout, slot_bytes, pool_stride,
    ExpertBank, LayerInputs, make_layer, make_bank, bf16_round, bf16_bits_to_f64,
    layer_pool_bytes, zipf_prior, encode_slot, INT4_GROUP, router_inputs, step_tokens,
)
from .exact import make_integer_layer, integer_weights, IntegerBank  # noqa: F401
