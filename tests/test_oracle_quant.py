"""Pins of the oracle's quantizers and dequantizer (CPU only).

Each pin comes from outside the oracle: a group worked by hand from the
ExactMoE section 3.2 equation, the rounding-error bound that equation implies,
idempotence, and the section 3.2 memory equation.
"""

import json
import os

import numpy as np
import pytest

import oracle
from inputs import f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _row(head, width=128):
    w = np.zeros(width, dtype=np.float32)
    w[: len(head)] = head
    return w


def test_int4_handworked_group():
    g = json.load(open(os.path.join(GOLD, "int4_group_handworked.json")))
    w = _bf16(_row(g["w_head"]))[None, :]
    q, s = oracle.quantize_int4_g128(w)
    assert s.dtype == np.float16 and s.shape == (1, 1)
    assert float(s[0, 0]) == g["scale"]
    assert q[0, :4].tolist() == g["q_head"]
    assert not q[0, 4:].any()
    assert q[0, :4].tolist() != g["half_away_from_zero_would_give"]
    w_hat = oracle.dequantize(oracle.TIER_INT4, q, s)
    assert w_hat[0, :4].tolist() == g["w_hat_head"]
    # the error at the two exact ties is exactly s/2
    err = np.abs(oracle.bf16_bits_to_f32(w).astype(np.float64) - w_hat)
    assert err[0, 1] == g["scale"] / 2 and err[0, 3] == g["scale"] / 2


def test_int8_handworked_row():
    g = json.load(open(os.path.join(GOLD, "int8_row_handworked.json")))
    w = _bf16(_row(g["w_head"]))[None, :]
    q, s = oracle.quantize_int8_per_channel(w)
    assert float(s[0]) == g["scale"]
    assert q[0, :4].tolist() == g["q_head"]
    assert not q[0, 4:].any()


def _random_weight(rng, n, k, std=0.02):
    return _bf16(rng.standard_normal((n, k)).astype(np.float32) * std)


@pytest.mark.parametrize("std", [0.02, 1.0, 3e-3])
def test_int4_roundtrip_bound_and_extremes(std):
    rng = np.random.default_rng(1)
    w = _random_weight(rng, 64, 512, std)
    q, s = oracle.quantize_int4_g128(w)
    wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
    w_hat = oracle.dequantize(2, q, s)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    # |w - q s| <= s/2 up to the fp32 rounding of w/s (|w/s| < 7.5 => 2^-20 rel)
    assert np.all(np.abs(wf - w_hat) <= s64 / 2 * (1 + 2.0 ** -20))
    # the scale is max/7 rounded once to fp16 (nearest): relative error <= 2^-11
    m = np.abs(wf).reshape(64, 4, 128).max(axis=2)
    assert np.all(np.abs(s.astype(np.float64) - m / 7) <= (m / 7) * 2.0 ** -11 * (1 + 1e-6))
    # the element of largest magnitude maps to +-7, and -8 never occurs
    qa = q.reshape(64, 4, 128)
    wa = wf.reshape(64, 4, 128)
    idx = np.abs(wa).argmax(axis=2)
    top_q = np.take_along_axis(qa, idx[:, :, None], axis=2)[..., 0]
    top_w = np.take_along_axis(wa, idx[:, :, None], axis=2)[..., 0]
    assert np.all(top_q == 7 * np.sign(top_w))
    assert q.min() >= -7 and q.max() <= 7


def test_int8_roundtrip_bound():
    rng = np.random.default_rng(2)
    w = _random_weight(rng, 48, 384)
    q, s = oracle.quantize_int8_per_channel(w)
    wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
    w_hat = oracle.dequantize(1, q, s)
    assert np.all(np.abs(wf - w_hat) <= s.astype(np.float64)[:, None] / 2 * (1 + 2.0 ** -16))
    top = np.abs(wf).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(48), top]) == 127)


@pytest.mark.parametrize("tier", [1, 2])
def test_idempotence(tier):
    """Quantizing the dequantized weights reproduces the same codes and scales.

    Every group's extreme element is exactly +-7 s (or +-127 s), so max/7 gives
    back s; the codes are then exact integers.  Values must be bf16-exact for
    this to hold, which they are for these small code * power-of-two scales.
    """
    rng = np.random.default_rng(3)
    if tier == 2:
        q0 = rng.integers(-7, 8, size=(32, 256)).astype(np.int8)
        q0[:, ::128] = 7                      # each group has a +7 entry
        s0 = (2.0 ** rng.integers(-12, -4, size=(32, 2))).astype(np.float16)
        w = oracle.dequantize(2, q0, s0)
    else:
        q0 = rng.integers(-127, 128, size=(16, 256)).astype(np.int8)
        q0[:, 0] = -127
        s0 = (2.0 ** rng.integers(-14, -8, size=16)).astype(np.float16)
        w = oracle.dequantize(1, q0, s0)
    w_bf16 = f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f32(w_bf16).astype(np.float64), w)
    q1, s1 = oracle.quantize_tier(tier, w_bf16)
    assert np.array_equal(q1, q0) and np.array_equal(s1, s0)


def test_zero_group_and_errors():
    w = np.zeros((2, 256), dtype=np.uint16)
    w[1, 200] = _bf16([0.5])[0]
    q, s = oracle.quantize_int4_g128(w)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and not q[0].any()
    assert q[1, 200] == 7
    bad = w.copy()
    bad[0, 3] = 0x7FC0                         # NaN
    with pytest.raises(ValueError):
        oracle.quantize_int4_g128(bad)
    big = np.zeros((1, 128), dtype=np.uint16)
    big[0, 0] = _bf16([1.0e6])[0]              # 1e6/7 > 65504: fp16 overflow
    with pytest.raises(ValueError):
        oracle.quantize_int4_g128(big)
    with pytest.raises(ValueError):
        oracle.quantize_int8_per_channel(big * 0 + _bf16([1.0e7])[0])


@pytest.mark.parametrize("n,k", [(1536, 2048), (2048, 768), (28672, 4096)])
def test_memory_equation(n, k):
    """ExactMoE section 3.2 memory equation: M = P (4/8 + 16/(128*8)) bytes."""
    P = n * k
    assert oracle.layout.payload_size(2, n, k) * 1024 == P * (512 + 16)
    assert oracle.packed_size(2, n, k) % 256 == 0
    assert oracle.packed_size(2, n, k) - oracle.layout.payload_size(2, n, k) < 256


def test_bf16_rounding_helpers():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20,
                     3.0e38, 1e-40], dtype=np.float32)
    out = oracle.f32_to_bf16_rne(vals)
    # ties to even: 1+2^-8 -> 1.0 ; 1+3*2^-8 -> 1+2^-6 ; above the tie rounds up
    exp = [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]
    assert out[:5].tolist() == exp
    import torch
    t = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, t)
    assert np.array_equal(oracle.bf16_bits_to_f32(np.array([0x3F80, 0xC020], np.uint16)),
                          np.array([1.0, -2.5], np.float32))
