"""CPU oracle for the quantized MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow numpy code that states what the layer computes, step by step, in
float64 wherever the pages do not fix a precision.  It is imported only by the
test suite, by the package's smoke check and by the benchmark's CPU-baseline
leg; the product path never calls it and has no fallback to it.

It shares no code with the HIP library: it has its own bf16/fp16 rounding, its
own quantizer and its own writer of the packed byte layout.  Its only shared
dependency is the seeded input generator package (`inputs`), which holds none
of the layer's arithmetic.
"""

from .moe_oracle import (  # noqa: F401
    TIER_BF16,
    TIER_INT8,
    TIER_INT4,
    make_expert,
    OracleExpert,
    bf16_bits_to_f32,
    f32_to_bf16_rne,
    quantize_int4_g128,
    quantize_int8_per_channel,
    dequantize,
    quantize_tier,
    router_logits,
    select_topk,
    gate_weights,
    permutation,
    expert_ffn,
    layer_forward,
    wave_forward,
    plan_tiers,
    route,
    OracleLayer,
)
from . import layout  # noqa: F401
from .layout import packed_size, pack_matrix, LAYOUT_PLAIN, LAYOUT_GATE_UP  # noqa: F401
