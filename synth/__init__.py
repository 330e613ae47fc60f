"""Seeded synthetic inputs for the low-bit MoE FFN layer.

This package only *makes inputs*: token activations, router logits and
expert weights stored in the packed low-bit format the layer consumes.
It holds none of the layer's arithmetic (no routing, no permutation, no
activation quantization, no projections); both the CPU oracle and the GPU
library are fed from here and never from each other.
"""
from .gen import (CONFIGS, LAYERS, LayerConfig, make_layer, config_by_id,  # noqa: F401
                  pack_codes, quantize_matrix, bf16_bits_from_f32,
                  with_random_codes, with_x_rows)
