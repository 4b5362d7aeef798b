"""Seeded synthetic inputs for the routed MoE layer.

This package is shared by the CPU oracle's tests and the HIP path's tests and
bench.  It makes inputs only: router matrices, packed block-quantised expert
weights (the "checkpoint" a serving engine would load) and bf16 hidden
states.  It computes no part of the layer forward; the logits it evaluates
in fp64 serve only to reject token draws whose top-k would be a near tie.
"""
from .layers import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    Layer,
    QWeight,
    make_layer,
    make_tokens,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    quantize_mxfp4,
    quantize_nvfp4,
    quantize_fp8,
    e2m1_encode,
    e4m3_encode,
)
from .crafted import CRAFTED, WIDE, crafted_layer, crafted_tokens  # noqa: F401,E402
