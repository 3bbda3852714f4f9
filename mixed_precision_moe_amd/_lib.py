"""ctypes loader of libmoe.so (the C ABI declared in include/moe.h).

The library is loaded from this package directory only.  There is no
fallback: if it is missing, importing the binding raises, so nothing can run
the layer anywhere but in the HIP kernels.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

# status codes (moe_status)
MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_ERANGE, MOE_ENOSPC, MOE_EHIP = range(6)
TIER_BF16, TIER_INT8, TIER_INT4 = 0, 1, 2
LAYOUT_PLAIN, LAYOUT_GATE_UP = 0, 1
DTYPE_BF16, DTYPE_F32 = 0, 1
PATH_DECODE, PATH_LARGE_BATCH = 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES
ROUTER_AUTO, ROUTER_CANONICAL, ROUTER_MFMA = 0, 1, 2

# every symbol include/moe.h declares
EXPORTS = (
    "moe_packed_size", "moe_quantize_pack", "moe_quantize_pack_async", "moe_layer_create",
    "moe_layer_set_experts", "moe_layer_set_slots", "moe_layer_set_slot_map",
    "moe_layer_set_hotness", "moe_plan_tiers", "moe_layer_destroy", "moe_workspace_size",
    "moe_route", "moe_layer_forward", "moe_layer_forward_wave", "moe_layer_set_stage_events",
    "moe_layer_set_router_mode", "moe_strerror", "moe_last_error", "moe_abi_version",
    "moe_unpack_codes", "moe_layer_plan", "moe_layer_forward_noalloc",
)


class ExpertHandle(ctypes.Structure):
    _fields_ = [("tier", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m mixed_precision_moe_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_packed_size": (sz, [ctypes.c_int, i64, i64]),
        "moe_quantize_pack": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, vp, i64, i64, vp, sz, vp]),
        "moe_layer_create": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(ExpertHandle),
                                            vp, ctypes.POINTER(vp)]),
        "moe_layer_set_experts": (ctypes.c_int, [vp, i32, i32, ctypes.POINTER(ExpertHandle), vp]),
        "moe_quantize_pack_async": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, vp, i64, i64, vp, sz,
                                                   vp, vp]),
        "moe_layer_set_hotness": (ctypes.c_int, [vp, vp, ctypes.c_float]),
        "moe_plan_tiers": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(sz), sz,
                                          i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "moe_layer_set_slots": (ctypes.c_int, [vp, i32, i32, ctypes.POINTER(ExpertHandle), vp]),
        "moe_layer_set_slot_map": (ctypes.c_int, [vp, ctypes.POINTER(i32), vp]),
        "moe_layer_destroy": (ctypes.c_int, [vp]),
        "moe_workspace_size": (sz, [vp, i32]),
        "moe_route": (ctypes.c_int, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_layer_forward": (ctypes.c_int, [vp, vp, vp, vp, i32, vp, ctypes.c_int, vp, sz, vp]),
        "moe_layer_forward_wave": (ctypes.c_int, [vp, vp, vp, vp, i32, vp, ctypes.c_int, ctypes.c_int,
                                                  vp, sz, vp]),
        "moe_layer_set_stage_events": (ctypes.c_int, [vp, ctypes.POINTER(vp), i32]),
        "moe_layer_set_router_mode": (ctypes.c_int, [vp, i32]),
        "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (ctypes.c_int, []),
        "moe_unpack_codes": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, vp, sz, i64, i64, vp, vp]),
        "moe_layer_plan": (ctypes.c_int, [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                          ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "moe_layer_forward_noalloc": (ctypes.c_int, [vp, vp, vp, vp, i32, vp, ctypes.c_int, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        lib = load()
        msg = lib.moe_last_error().decode(errors="replace") or lib.moe_strerror(status).decode()
        raise MoeError(status, where, msg)
