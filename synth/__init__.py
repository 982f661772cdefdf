"""Seeded synthetic MoE layers and token batches.

This module only draws numbers: shapes, distributions, seeds, bf16 rounding of
the draws, the int8 per-output-channel and int4 group-wise quantisation of
expert weights, and the int4 storage encoding (two values per byte). It
holds none of the layer's forward arithmetic, and it is the one module that both
the CPU oracle (via the tests) and the GPU binding consume.
"""
from .configs import CONFIGS, LayerConfig, get_config
from .generate import (make_layer, make_tokens, make_routing, zipf_bias, quantize_per_out_channel,
                       quantize_int4_groupwise, pack_int4_pairs, INT4_GROUP, SynthLayer, layer_kwargs)

__all__ = ["CONFIGS", "LayerConfig", "get_config", "make_layer", "make_tokens", "make_routing", "zipf_bias",
           "quantize_per_out_channel", "quantize_int4_groupwise", "pack_int4_pairs", "INT4_GROUP", "SynthLayer", "layer_kwargs"]
