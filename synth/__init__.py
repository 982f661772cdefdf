"""Seeded synthetic MoE layers and token batches.

This module only draws numbers: shapes, distributions, seeds, bf16 rounding of
the draws and the int8 per-output-channel quantisation of expert weights. It
holds none of the layer's forward arithmetic, and it is the one module that both
the CPU oracle (via the tests) and the GPU binding consume.
"""
from .configs import CONFIGS, LayerConfig, get_config
from .generate import make_layer, make_tokens, make_routing, zipf_bias, quantize_per_out_channel, SynthLayer

__all__ = ["CONFIGS", "LayerConfig", "get_config", "make_layer", "make_tokens", "make_routing", "zipf_bias",
           "quantize_per_out_channel", "SynthLayer"]
