"""The library's host reader of the packed layout against the oracle's packer
(CPU only, no GPU call).

ExactMoE §3.3 stores every routed expert once in the kernel's own format:
packed gate/up codes, packed down codes and FP16 scales.  Here the oracle
quantizes seeded master weights (§3.2 quantizer) and writes the layout with its
own packer (oracle/layout.py); moe_unpack_codes, the library's independent
inverse of that layout, must return exactly the oracle's codes and scales, for
every tier and both row orders, at the Qwen3-30B-A3B and Mixtral shapes.
"""

import ctypes
import os

import numpy as np
import pytest

import inputs
import oracle
from mixed_precision_moe_amd import _lib
from oracle import layout

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libmoe.so not built (run __graft_entry__.build())")


def _master(shape, seed):
    rng = np.random.default_rng([7, seed, *shape])
    return inputs.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02))


def _unpack(tier, lay, blob, n, k):
    lib = _lib.load()
    q = np.full((n, k), 99, dtype=np.int8)
    if tier == oracle.TIER_INT4:
        aux = np.zeros((n, k // 128), dtype=np.uint16)
    elif tier == oracle.TIER_INT8:
        aux = np.zeros(n, dtype=np.uint16)
    else:
        aux = np.zeros((n, k), dtype=np.uint16)
    rc = lib.moe_unpack_codes(tier, lay, blob.ctypes.data, blob.nbytes, n, k,
                              q.ctypes.data if tier != oracle.TIER_BF16 else None, aux.ctypes.data)
    assert rc == _lib.MOE_OK, lib.moe_last_error()
    return q, aux


def _check(tier, lay, w):
    n, k = w.shape
    q, s = oracle.quantize_tier(tier, w)
    blob = layout.pack_matrix(tier, lay, q=q, s=s, w_bf16=w)
    gq, gaux = _unpack(tier, lay, blob, n, k)
    if tier == oracle.TIER_BF16:
        assert np.array_equal(gaux, w)
    else:
        assert np.array_equal(gq, q)
        assert np.array_equal(gaux, s.view(np.uint16))


# (n_out, k_in) of the gate/up [2I, H] and down [H, I] matrices
QWEN30B = [((1536, 2048), layout.LAYOUT_GATE_UP), ((2048, 768), layout.LAYOUT_PLAIN)]
MIXTRAL = [((28672, 4096), layout.LAYOUT_GATE_UP), ((4096, 14336), layout.LAYOUT_PLAIN)]


@pytest.mark.parametrize("tier", [oracle.TIER_BF16, oracle.TIER_INT8, oracle.TIER_INT4])
@pytest.mark.parametrize("shape,lay", QWEN30B)
def test_unpack_qwen30b_shapes(tier, shape, lay):
    _check(tier, lay, _master(shape, tier))


@pytest.mark.parametrize("shape,lay", MIXTRAL)
def test_unpack_mixtral_shapes_int4(shape, lay):
    _check(oracle.TIER_INT4, lay, _master(shape, 2))


@pytest.mark.parametrize("tier", [oracle.TIER_BF16, oracle.TIER_INT8, oracle.TIER_INT4])
def test_unpack_layer_expert_from_the_workload(tier):
    """One real expert of the Qwen3-30B-shaped workload: gate and up packed as
    one fused matrix come back as [W_g; W_u] in source row order."""
    wg, wu, wd = inputs.gen_expert(inputs.get_config(2), 3)
    _check(tier, layout.LAYOUT_GATE_UP, np.concatenate([wg, wu], axis=0))
    _check(tier, layout.LAYOUT_PLAIN, wd)


def test_unpack_edge_codes():
    """Extreme codes and scales survive the round trip: -8 and 7 (int4),
    -128 and 127 (int8), zero groups, a subnormal fp16 scale."""
    n, k = 64, 256
    q4 = np.tile(np.array([-8, 7, 0, -1, 1, 3, -4, 5], np.int8), (n, k // 8))
    s4 = np.zeros((n, k // 128), np.float16)
    s4[:, 0] = np.float16(0.125)
    s4[1, 1] = np.float16(2.0 ** -24)            # smallest fp16 subnormal
    blob = layout.pack_matrix(oracle.TIER_INT4, layout.LAYOUT_PLAIN, q=q4, s=s4)
    gq, gs = _unpack(oracle.TIER_INT4, layout.LAYOUT_PLAIN, blob, n, k)
    assert np.array_equal(gq, q4) and np.array_equal(gs, s4.view(np.uint16))
    q8 = np.tile(np.array([-128, 127, 0, -1], np.int8), (n, k // 4))
    s8 = np.linspace(0, 1, n).astype(np.float16)
    blob = layout.pack_matrix(oracle.TIER_INT8, layout.LAYOUT_GATE_UP, q=q8, s=s8)
    gq, gs = _unpack(oracle.TIER_INT8, layout.LAYOUT_GATE_UP, blob, n, k)
    assert np.array_equal(gq, q8) and np.array_equal(gs, s8.view(np.uint16))


def test_unpack_validation():
    lib = _lib.load()
    buf = np.zeros(1 << 16, np.uint8)
    q = np.zeros(64 * 128, np.int8)
    aux = np.zeros(64 * 128, np.uint16)
    f = lib.moe_unpack_codes
    assert f(3, 0, buf.ctypes.data, buf.nbytes, 64, 128, q.ctypes.data, aux.ctypes.data) == _lib.MOE_EINVAL
    assert f(2, 5, buf.ctypes.data, buf.nbytes, 64, 128, q.ctypes.data, aux.ctypes.data) == _lib.MOE_EINVAL
    assert f(2, 0, None, buf.nbytes, 64, 128, q.ctypes.data, aux.ctypes.data) == _lib.MOE_EINVAL
    assert f(2, 0, buf.ctypes.data, buf.nbytes, 64, 128, None, aux.ctypes.data) == _lib.MOE_EINVAL
    assert f(2, 0, buf.ctypes.data, buf.nbytes, 64, 100, q.ctypes.data, aux.ctypes.data) == _lib.MOE_ESHAPE
    assert f(2, 0, buf.ctypes.data, buf.nbytes, 48, 128, q.ctypes.data, aux.ctypes.data) == _lib.MOE_ESHAPE
    need = layout.payload_size(2, 64, 128)
    assert f(2, 0, buf.ctypes.data, need - 1, 64, 128, q.ctypes.data, aux.ctypes.data) == _lib.MOE_ENOSPC
    assert b"needs" in lib.moe_last_error()
    assert f(0, 0, buf.ctypes.data, buf.nbytes, 64, 128, None, aux.ctypes.data) == _lib.MOE_OK
    assert lib.moe_last_error() == b""
