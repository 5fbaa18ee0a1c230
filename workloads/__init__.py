"""Seeded synthetic inputs for the MoE expert-layer forward.

This package only draws random numbers and stores them in the dtypes the
layer consumes. It holds none of the layer's arithmetic (no routing, no
softmax, no top-K, no GEMM), so both the CPU oracle and the HIP path can take
their inputs from it without sharing any part of the computation.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    EPShareWorkload,
    LayerWorkload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_ep_share,
    make_config,
    make_layer,
    make_micro_batch,
    random_bf16_matrix,
    zipf_bias,
)
