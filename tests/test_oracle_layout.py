"""Pins of the oracle's packed-layout writer (CPU only).

The layout is this project's own specification (stated in oracle/layout.py).
Here every sampled element is located by scalar arithmetic written straight
from that text and decoded from the blob, so a wrong stride, nibble position,
row interleave or scale index in the vectorized writer fails.
"""

import numpy as np
import pytest

import oracle
from oracle.layout import LAYOUT_GATE_UP, LAYOUT_PLAIN, TIER_BF16, TIER_INT4, TIER_INT8


def _source_row(p, n, layout):
    if layout == LAYOUT_PLAIN:
        return p
    b, w = divmod(p, 64)
    return 32 * b + w if w < 32 else n // 2 + 32 * b + (w - 32)


def _coords(p, k, K):
    """packed row p, column k -> (block index, strip-in-quad, lane, step, element)."""
    G = K // 128
    t, r = divmod(p, 16)
    Q, u = divmod(t, 4)
    g, kk = divmod(k, 128)
    s, rem = divmod(kk, 32)
    c, i = divmod(rem, 8)
    return Q * G + g, u, 16 * c + r, s, i


def _decode(blob, tier, p, k, N, K):
    block, u, lane, s, i = _coords(p, k, K)
    r = p % 16
    if tier == TIER_INT4:
        base = block * 4224
        word_at = base + 1024 * u + 16 * lane + 4 * s
        word = int.from_bytes(bytes(blob[word_at:word_at + 4]), "little")
        nib = (i // 2) + 4 * (i % 2)
        q = ((word >> (4 * nib)) & 0xF) - 8
        sa = base + 4096 + 2 * (4 * r + u)
        sc = np.frombuffer(bytes(blob[sa:sa + 2]), dtype="<f2")[0]
        return q, sc
    if tier == TIER_INT8:
        at = block * 8192 + 2048 * u + (s // 2) * 1024 + 16 * lane + 8 * (s % 2) + i
        q = int(blob[at]) - 128
        Q = p // 64
        sa = N * K + 2 * (64 * Q + 4 * r + u)
        return q, np.frombuffer(bytes(blob[sa:sa + 2]), dtype="<f2")[0]
    at = block * 16384 + 4096 * u + s * 1024 + 16 * lane + 2 * i
    return int.from_bytes(bytes(blob[at:at + 2]), "little"), None


@pytest.mark.parametrize("tier", [TIER_INT4, TIER_INT8, TIER_BF16])
@pytest.mark.parametrize("layout", [LAYOUT_PLAIN, LAYOUT_GATE_UP])
def test_layout_scalar_decode(tier, layout):
    rng = np.random.default_rng(31)
    N, K = 128, 384
    if tier == TIER_BF16:
        w = rng.integers(0, 65536, size=(N, K)).astype(np.uint16)
        blob = oracle.pack_matrix(tier, layout, w_bf16=w)
    else:
        lo, hi = (-8, 8) if tier == TIER_INT4 else (-128, 128)
        q = rng.integers(lo, hi, size=(N, K)).astype(np.int8)
        s = rng.standard_normal((N, K // 128) if tier == TIER_INT4 else N).astype(np.float16)
        blob = oracle.pack_matrix(tier, layout, q=q, s=s)
    assert blob.size == oracle.packed_size(tier, N, K)
    for _ in range(600):
        p, k = int(rng.integers(N)), int(rng.integers(K))
        src = _source_row(p, N, layout)
        val, sc = _decode(blob, tier, p, k, N, K)
        if tier == TIER_BF16:
            assert val == w[src, k]
        else:
            assert val == q[src, k]
            want = s[src, k // 128] if tier == TIER_INT4 else s[src]
            assert sc == want
    # padding beyond the payload is zero
    assert not blob[oracle.layout.payload_size(tier, N, K):].any()


def test_gate_up_interleave_pairs():
    """In the gate/up layout, packed rows 64b+w and 64b+32+w hold gate and up of
    the same intermediate channel 32b+w."""
    n = 256
    for p in range(0, n, 64):
        for w in range(32):
            g = _source_row(p + w, n, LAYOUT_GATE_UP)
            u = _source_row(p + 32 + w, n, LAYOUT_GATE_UP)
            assert u == g + n // 2
    assert sorted(_source_row(p, n, LAYOUT_GATE_UP) for p in range(n)) == list(range(n))
    assert np.array_equal(oracle.layout.packed_row_source(n, LAYOUT_GATE_UP),
                          [_source_row(p, n, LAYOUT_GATE_UP) for p in range(n)])


def test_layout_rejects_bad_shapes():
    q = np.zeros((64, 100), np.int8)
    with pytest.raises(ValueError):
        oracle.pack_matrix(TIER_INT8, LAYOUT_PLAIN, q=q, s=np.zeros(64, np.float16))
    q = np.zeros((48, 128), np.int8)
    with pytest.raises(ValueError):
        oracle.pack_matrix(TIER_INT8, LAYOUT_PLAIN, q=q, s=np.zeros(48, np.float16))
    q = np.zeros((96, 128), np.int8)
    with pytest.raises(ValueError):
        oracle.pack_matrix(TIER_INT8, LAYOUT_GATE_UP, q=q, s=np.zeros(48, np.float16))
