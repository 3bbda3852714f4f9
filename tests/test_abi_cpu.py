"""The C ABI library loads and exports what include/moe.h declares; host-side
validation rejects bad arguments before any HIP call (CPU only: no call here
reaches the GPU)."""

import ctypes
import os
import re

import pytest

import oracle
from mixed_precision_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")



def _gpu_visible() -> bool:
    """Whether this process can see a GPU.  torch's device count on ROCm reads
    the device list without starting the HIP runtime."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The validation tests below pass addresses that are never dereferenced only
# because host-side validation rejects the call first; on a machine with a GPU
# a regression there could launch a kernel on them, so they run where no GPU
# is visible (the GPU tests cover the same entry points with real buffers).
pytestmark = [
    pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                       reason="libmoe.so not built (run __graft_entry__.build())"),
    pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: CPU-only machine"),
]


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)
    assert lib.moe_abi_version() == 1


def test_packed_size_matches_layout_spec():
    lib = _lib.load()
    for tier in (0, 1, 2):
        for n, k in [(64, 128), (1536, 2048), (2048, 768), (28672, 4096), (4096, 14336),
                     (1024, 2048), (192, 256)]:
            assert lib.moe_packed_size(tier, n, k) == oracle.packed_size(tier, n, k)
    for n, k in [(64, 100), (10, 128), (16, 128), (48, 128), (0, 128), (64, 0), (-64, 128)]:
        assert lib.moe_packed_size(2, n, k) == 0
    assert lib.moe_packed_size(3, 64, 128) == 0


def test_strerror_and_last_error():
    lib = _lib.load()
    for code in range(6):
        assert lib.moe_strerror(code)
    assert lib.moe_strerror(99) == b"unknown status"


FAKE = 0x100000   # a 256-aligned address that is never dereferenced


def test_quantize_pack_validation():
    lib = _lib.load()
    q = lib.moe_quantize_pack
    assert q(5, 0, FAKE, 64, 128, FAKE, 1 << 20, None) == _lib.MOE_EINVAL      # tier
    assert q(2, 7, FAKE, 64, 128, FAKE, 1 << 20, None) == _lib.MOE_EINVAL      # layout
    assert q(2, 0, None, 64, 128, FAKE, 1 << 20, None) == _lib.MOE_EINVAL      # null w
    assert q(2, 0, FAKE, 64, 128, FAKE + 16, 1 << 20, None) == _lib.MOE_EINVAL  # dst align
    assert q(2, 0, FAKE + 2, 64, 128, FAKE, 1 << 20, None) == _lib.MOE_EINVAL  # w align
    assert q(2, 0, FAKE, 64, 100, FAKE, 1 << 20, None) == _lib.MOE_ESHAPE
    assert q(2, 0, FAKE, 16, 128, FAKE, 1 << 20, None) == _lib.MOE_ESHAPE     # quads of 64 rows
    assert q(2, 1, FAKE, 48, 128, FAKE, 1 << 20, None) == _lib.MOE_ESHAPE
    assert q(0, 0, FAKE, 1 << 16, 1 << 15, FAKE, 1 << 40, None) == _lib.MOE_ESHAPE   # >= 4 GiB
    need = lib.moe_packed_size(2, 64, 128)
    assert q(2, 0, FAKE, 64, 128, FAKE, need - 1, None) == _lib.MOE_ENOSPC
    assert b"needed" in lib.moe_last_error()


def _handles(n, tier=2, w13=FAKE, w2=FAKE):
    arr = (_lib.ExpertHandle * n)()
    for i in range(n):
        arr[i] = _lib.ExpertHandle(tier, 0, w13, w2)
    return arr


@pytest.mark.parametrize("desc,status", [
    ((255, 512, 8, 2), _lib.MOE_ESHAPE),     # H % 256
    ((256, 500, 8, 2), _lib.MOE_ESHAPE),     # I % 128
    ((256, 512, 0, 1), _lib.MOE_ESHAPE),     # E
    ((256, 512, 1025, 2), _lib.MOE_ESHAPE),  # E too large
    ((256, 512, 8, 9), _lib.MOE_ESHAPE),     # k > E
    ((256, 512, 32, 17), _lib.MOE_ESHAPE),   # k > 16
    ((256, 512, 8, 0), _lib.MOE_ESHAPE),     # k = 0
])
def test_layer_create_rejects_bad_geometry(desc, status):
    lib = _lib.load()
    d = _lib.LayerDesc(*desc)
    out = ctypes.c_void_p()
    n = max(1, min(desc[2], 2048))
    assert lib.moe_layer_create(ctypes.byref(d), _handles(n), None, ctypes.byref(out)) == status
    assert not out.value


def test_layer_create_rejects_bad_handles():
    lib = _lib.load()
    d = _lib.LayerDesc(256, 512, 4, 2)
    out = ctypes.c_void_p()
    for bad in (_handles(4, tier=3), _handles(4, w13=0), _handles(4, w2=FAKE + 64)):
        assert lib.moe_layer_create(ctypes.byref(d), bad, None, ctypes.byref(out)) == _lib.MOE_EINVAL
    assert lib.moe_layer_create(None, _handles(4), None, ctypes.byref(out)) == _lib.MOE_EINVAL


def test_null_layer_calls():
    lib = _lib.load()
    assert lib.moe_workspace_size(None, 8) == 0
    assert lib.moe_layer_destroy(None) == _lib.MOE_EINVAL
    assert lib.moe_layer_forward(None, FAKE, FAKE, None, 4, FAKE, 1, FAKE, 1 << 20, None) == _lib.MOE_EINVAL
    assert lib.moe_route(None, FAKE, FAKE, None, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                         1 << 20, None) == _lib.MOE_EINVAL
    assert lib.moe_layer_set_stage_events(None, None, 0) == _lib.MOE_EINVAL
    assert lib.moe_layer_set_router_mode(None, _lib.ROUTER_AUTO) == _lib.MOE_EINVAL
    assert lib.moe_layer_set_slots(None, 0, 1, _handles(1), None) == _lib.MOE_EINVAL
    assert lib.moe_layer_set_slot_map(None, (ctypes.c_int32 * 4)(-1, -1, -1, -1), None) == _lib.MOE_EINVAL
    assert lib.moe_layer_forward_wave(None, FAKE, FAKE, None, 4, FAKE, 1, 1, FAKE, 1 << 20,
                                      None) == _lib.MOE_EINVAL


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    """The binding has no fallback: a missing library is an import-time error.
    (monkeypatch restores the loaded library afterwards.)"""
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()
