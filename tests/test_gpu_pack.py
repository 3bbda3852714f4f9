"""GPU quantize-pack vs the oracle's quantizer and independent layout writer:
bytes must be identical (codes, fp16 scales, padding)."""

import numpy as np
import pytest

import inputs
import oracle
from tests._harness import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import mixed_precision_moe_amd as mm
    import torch
    assert torch.cuda.is_available()
    return mm


def _oracle_blob(tier, layout, w):
    if tier == oracle.TIER_BF16:
        return oracle.pack_matrix(tier, layout, w_bf16=w)
    q, s = oracle.quantize_tier(tier, w)
    return oracle.pack_matrix(tier, layout, q=q, s=s)


@pytest.mark.parametrize("tier", [2, 1, 0])
@pytest.mark.parametrize("cid", [1, 2])
def test_pack_bytes_match_oracle(mm, tier, cid):
    cfg = inputs.get_config(cid)
    wg, wu, wd = inputs.gen_expert(cfg, 3)
    w13 = np.concatenate([wg, wu], axis=0)
    for layout, w in ((mm.LAYOUT_GATE_UP, w13), (mm.LAYOUT_PLAIN, wd)):
        log(f"pack cfg{cid} tier {tier} layout {layout} shape {w.shape}")
        blob = mm.quantize_pack(to_dev(w), tier, layout).cpu().numpy()
        ref = _oracle_blob(tier, layout, w)
        assert blob.size == ref.size
        bad = np.nonzero(blob != ref)[0]
        assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_pack_edge_values(mm):
    """Exact halves (ties to even), zero groups, tiny (subnormal fp16) scales,
    a group whose extreme is negative, and values near the fp16 scale limit."""
    rng = np.random.default_rng(7)
    n, k = 64, 512
    w = rng.standard_normal((n, k)).astype(np.float32) * 0.02
    w[0, :128] = 0.0                                    # zero group
    w[1, :128] = 0.0
    w[1, :4] = [0.875, -0.4375, 0.0625, 0.3125]         # hand-worked halves
    w[2, 128:256] *= 1e-4                               # subnormal fp16 scale
    w[3, 256:384] = -np.abs(w[3, 256:384])              # all negative
    w[4, :] = 400000.0 * np.sign(w[4, :])               # scale 57142: close to fp16 max
    w[5, 384:] = rng.integers(-7, 8, size=128) * 0.125  # exact multiples of the scale
    w[5, 384] = 0.875
    wb = inputs.f32_to_bf16_bits(w)
    for tier in (2, 1):
        for layout in (mm.LAYOUT_PLAIN, mm.LAYOUT_GATE_UP):
            blob = mm.quantize_pack(to_dev(wb), tier, layout).cpu().numpy()
            assert np.array_equal(blob, _oracle_blob(tier, layout, wb)), (tier, layout)


def test_pack_errors(mm):
    w = np.zeros((64, 128), np.uint16)
    w[3, 5] = 0x7FC0                                    # NaN
    with pytest.raises(mm.MoeError) as ei:
        mm.quantize_pack(to_dev(w), 2)
    assert ei.value.status == 3
    w[3, 5] = inputs.f32_to_bf16_bits(np.float32([1.0e6]))[0]   # 1e6/7 overflows fp16
    with pytest.raises(mm.MoeError) as ei:
        mm.quantize_pack(to_dev(w), 2)
    assert ei.value.status == 3
    # int8 of the same value is fine (1e6/127 < 65504)
    mm.quantize_pack(to_dev(w), 1)
    with pytest.raises(mm.MoeError) as ei:      # 16 rows: the layout packs quads of 64
        mm.quantize_pack(to_dev(w[:16]), 2)
    assert ei.value.status == 2
