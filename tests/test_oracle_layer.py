"""Pins of the oracle's expert FFN and combine (CPU only).

* E = 1, k = 1 reduces the layer to a dense SwiGLU FFN, checked against scalar
  Python loops (math.exp, torch's bf16 rounding) on a tiny size;
* the full pipeline on a tiny layer against per-token scalar loops;
* ExactMoE section 3.4: the outputs over disjoint expert subsets ("waves")
  sum to the full output, with router weights not renormalized per wave;
* permuting tokens permutes the outputs.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from inputs import f32_to_bf16_bits


def _bf16(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _f(u16):
    return oracle.bf16_bits_to_f32(u16).astype(np.float64)


def _torch_bf16_round(v: float) -> float:
    return float(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).float()[0])


def _scalar_ffn(x_row, wg, wu, wd):
    """Scalar loops: g, u, silu(g)*u rounded fp32->bf16, then W_d."""
    I, H = wg.shape
    a16 = []
    for i in range(I):
        g = sum(float(wg[i, h]) * float(x_row[h]) for h in range(H))
        u = sum(float(wu[i, h]) * float(x_row[h]) for h in range(H))
        a = g / (1.0 + math.exp(-g)) * u
        a16.append(_torch_bf16_round(float(np.float32(a))))
    return [sum(float(wd[o, i]) * a16[i] for i in range(I)) for o in range(wd.shape[0])]


def _tiny_layer(rng, H, I, E, tiers):
    experts = {}
    for e in range(E):
        wg = _bf16(rng.standard_normal((I, H)) * 0.05)
        wu = _bf16(rng.standard_normal((I, H)) * 0.05)
        wd = _bf16(rng.standard_normal((H, I)) * 0.05)
        experts[e] = (wg, wu, wd)
    return experts


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_single_expert_is_dense_swiglu(tier):
    rng = np.random.default_rng(21)
    H, I, T = 256, 128, 3
    (wg, wu, wd), = _tiny_layer(rng, H, I, 1, [tier]).values()
    x = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((1, H)) * 0.02)
    layer = oracle.OracleLayer(H, I, 1, 1, np.array([tier]), lambda e: (wg, wu, wd))
    y, r = layer.forward(x, wr)
    assert np.all(r["ids"] == 0) and np.all(r["weights"] == 1.0)
    ex = layer.expert(0)
    if tier == 0:     # bf16 tier: no quantization at all
        assert np.array_equal(ex.wg_hat, _f(wg)) and np.array_equal(ex.wd_hat, _f(wd))
    xf = _f(x)
    for t in range(T):
        ref = _scalar_ffn(xf[t], ex.wg_hat, ex.wu_hat, ex.wd_hat)
        assert np.allclose(y[t], ref, rtol=2e-6, atol=1e-6)


def test_full_pipeline_scalar_brute_force():
    rng = np.random.default_rng(22)
    H, I, E, k, T = 256, 128, 4, 2, 4
    tiers = np.array([2, 1, 0, 2])
    src = _tiny_layer(rng, H, I, E, tiers)
    x = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((E, H)) * 0.05)
    bias = np.array([0.0, 0.5, -0.25, 0.125], np.float32)
    layer = oracle.OracleLayer(H, I, E, k, tiers, lambda e: src[e])
    y, r = layer.forward(x, wr, bias)
    xf, wrf = _f(x), _f(wr)
    for t in range(T):
        z = [sum(xf[t, h] * wrf[e, h] for h in range(H)) + float(bias[e]) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-z[e], e))[:k]
        S = sorted(order)
        assert r["ids"][t].tolist() == S
        m = max(z[e] for e in S)
        ex = [math.exp(z[e] - m) for e in S]
        w = [v / sum(ex) for v in ex]
        assert np.allclose(r["weights"][t], w, atol=1e-6)
        out = [0.0] * H
        for j, e in enumerate(S):
            o = layer.expert(e)
            fe = _scalar_ffn(xf[t], o.wg_hat, o.wu_hat, o.wd_hat)
            out = [a + w[j] * b for a, b in zip(out, fe)]
        rms = math.sqrt(sum(v * v for v in out) / H)
        assert np.max(np.abs(y[t] - np.array(out))) <= 1e-5 * rms


def _layer_and_inputs(seed=23):
    rng = np.random.default_rng(seed)
    H, I, E, k, T = 256, 256, 8, 3, 24
    tiers = rng.integers(0, 3, size=E)
    src = _tiny_layer(rng, H, I, E, tiers)
    x = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((E, H)) * 0.05)
    return oracle.OracleLayer(H, I, E, k, tiers, lambda e: src[e]), x, wr


def test_wave_additivity():
    """Disjoint expert subsets: partial outputs (weights kept) sum to the full output."""
    layer, x, wr = _layer_and_inputs()
    y, r = layer.forward(x, wr)
    rng = np.random.default_rng(5)
    waves = np.array_split(rng.permutation(layer.E), 3)
    total = np.zeros_like(y, dtype=np.float64)
    for wave in waves:
        members = set(int(e) for e in wave)

        def get(e, members=members):
            ex = layer.expert(e)
            if e in members:
                return ex
            return oracle.OracleExpert(ex.tier, ex.wg_hat, ex.wu_hat, np.zeros_like(ex.wd_hat))
        total += oracle.layer_forward(x, r, get)
    rms = np.sqrt(np.mean(y.astype(np.float64) ** 2))
    assert np.max(np.abs(total - y)) <= 1e-6 * rms
    # renormalizing the weights inside a wave would break the identity
    assert not np.allclose(y, 0)


def test_wave_forward_partition_sums_to_layer():
    """wave_forward over a partition of the experts: the waves sum to the full
    output, an empty wave is zero, and a wave holding every expert equals it."""
    layer, x, wr = _layer_and_inputs()
    y, r = layer.forward(x, wr)
    rng = np.random.default_rng(9)
    waves = np.array_split(rng.permutation(layer.E), 4)
    total = sum(oracle.wave_forward(x, r, layer.expert, w).astype(np.float64) for w in waves)
    rms = np.sqrt(np.mean(y.astype(np.float64) ** 2))
    assert np.max(np.abs(total - y)) <= 1e-6 * rms
    assert not np.any(oracle.wave_forward(x, r, layer.expert, []))
    full = oracle.wave_forward(x, r, layer.expert, range(layer.E))
    assert np.max(np.abs(full - y)) <= 1e-6 * rms
    # a one-expert wave holds exactly that expert's weighted rows
    e0 = int(r["ids"][0, 0])
    one = oracle.wave_forward(x, r, layer.expert, [e0])
    rows = np.nonzero((r["ids"] == e0).any(axis=1))[0]
    others = np.setdiff1d(np.arange(x.shape[0]), rows)
    assert not np.any(one[others]) and np.all(np.any(one[rows] != 0, axis=1))


def test_token_permutation_equivariance():
    layer, x, wr = _layer_and_inputs(24)
    y, _ = layer.forward(x, wr)
    perm = np.random.default_rng(6).permutation(x.shape[0])
    y2, _ = layer.forward(x[perm], wr)
    assert np.array_equal(y2, y[perm])


def test_token_subset_matches_full():
    layer, x, wr = _layer_and_inputs(25)
    y, _ = layer.forward(x, wr)
    sub = [3, 0, 17, 9]
    ys, _ = layer.forward(x, wr, token_subset=sub)
    assert np.array_equal(ys, y[sub])
    ys2, _ = layer.forward(x, wr, token_subset=sub, keep=False)
    assert np.array_equal(ys2, y[sub])
