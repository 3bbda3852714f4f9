"""Seeded synthetic inputs for the quantized MoE layer.

This package only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no quantizer, no routing, no GEMM).  Both the oracle and the
GPU path read their inputs from here, so the two sides see identical bits.  The
hot-expert ranking of the mixed-precision workloads is a stored table
(hot_sets.json), written by tests/golden/make_hot_sets.py from the oracle.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    TIER_BF16,
    TIER_INT8,
    TIER_INT4,
    LayerConfig,
    get_config,
    gen_tokens,
    gen_router,
    gen_bias,
    gen_tiers,
    hot_order,
    gen_expert,
    f32_to_bf16_bits,
)
