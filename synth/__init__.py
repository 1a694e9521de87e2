"""Seeded synthetic inputs for the W4A4 + rank-r linear layer.

This module only draws random tensors with the layer shapes and value
distributions of the workloads (diffusion-transformer and LLM linear
layers); it holds none of the method's arithmetic.  Both the HIP path
(through its binding) and the CPU oracle consume the same bytes.
"""

from .generators import (  # noqa: F401
    LAYERS,
    LayerSpec,
    bf16_bits_to_f32,
    f16_bits_to_f32,
    f64_to_bf16_bits,
    f64_to_f16_bits,
    layer_spec,
    make_full_weight,
    make_layer,
    make_random_layer,
)
