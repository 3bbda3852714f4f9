"""MI355X-native quantized mixture-of-experts FFN layer.

The layer runs entirely in the HIP library libmoe.so (C ABI in include/moe.h):
top-k routing, grouping by expert, the fused gate/up grouped GEMM with SwiGLU,
the down grouped GEMM and the weighted combine, over experts held at bf16,
int8 or int4 precision.  This package is the Python binding (argument
marshalling) and the build script.
"""

from ._lib import LIB_PATH, MoeError, load  # noqa: F401
from .api import (  # noqa: F401
    LAYOUT_GATE_UP,
    LAYOUT_PLAIN,
    ROUTER_AUTO,
    ROUTER_CANONICAL,
    ROUTER_MFMA,
    TIER_BF16,
    TIER_INT4,
    TIER_INT8,
    Layer,
    pack_expert,
    packed_size,
    plan_tiers,
    quantize_pack,
    quantize_pack_async,
)
from .dynaexq import DynaExq  # noqa: F401
