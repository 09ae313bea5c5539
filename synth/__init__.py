"""Seeded synthetic inputs for the W4A16 routed-expert layer.

This module only draws random numbers and shapes them; it holds none of the
layer's arithmetic (no quantisation, no dequantisation, no GEMM, no combine).
Both the CPU oracle (``oracle/``) and the HIP path receive their inputs from
here, so the two sides see identical bits.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    LayerShape,
    seed_for,
    expert_weights,
    expert_weights_device,
    activations,
    router_logits,
    zipf_prior,
    linear_inputs,
    sampler_logits,
)
