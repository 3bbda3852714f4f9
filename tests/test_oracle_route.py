"""Pins of the oracle's routing: logits, top-k, weights, permutation (CPU only)."""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from inputs import f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "router_order.json")))["cases"],
                         ids=lambda c: c["name"])
def test_logit_order_handworked(case):
    H = case["hidden"]
    x = np.zeros((1, H), np.float32)
    w = np.zeros((1, H), np.float32)
    for h, v in case["x_nonzero"].items():
        x[0, int(h)] = v
    for h, v in case["w_nonzero"].items():
        w[0, int(h)] = v
    z = oracle.router_logits(_bf16(x), _bf16(w))
    assert z.dtype == np.float32
    assert float(z[0, 0]) == case["z"]
    exact = float((x.astype(np.float64) * w).sum())
    assert exact == case["z_exact"]


@pytest.mark.parametrize("T,E,H", [(5, 8, 256), (3, 16, 512), (2, 4, 2048)])
def test_logits_close_to_exact_dot(T, E, H):
    rng = np.random.default_rng(11)
    x = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((E, H)) * 0.02)
    b = rng.standard_normal(E).astype(np.float32)
    z = oracle.router_logits(x, wr, b).astype(np.float64)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    wf = oracle.bf16_bits_to_f32(wr).astype(np.float64)
    exact = xf @ wf.T
    mag = np.abs(xf) @ np.abs(wf).T
    # fp32 summation error bound: chains of H/32 adds + 5 fold levels + bias add
    bound = (H // 32 + 6) * 2.0 ** -24 * (mag + np.abs(b)[None, :]) * 1.01
    assert np.all(np.abs(z - (exact + b[None, :].astype(np.float64))) <= bound + 1e-30)
    # a dropped term or wrong index is far outside the bound
    assert (np.abs(xf[:, :1] * wf[:, :1].T) > bound).any()


def _brute_topk(z_row, k):
    """All k-subsets; keep those no outsider beats: (z_o > z_i) or tie with lower index."""
    E = len(z_row)
    winners = []
    for S in itertools.combinations(range(E), k):
        ok = True
        for i in S:
            for o in range(E):
                if o in S:
                    continue
                if z_row[o] > z_row[i] or (z_row[o] == z_row[i] and o < i):
                    ok = False
        if ok:
            winners.append(list(S))
    return winners


def test_topk_brute_force_and_ties():
    rng = np.random.default_rng(12)
    for trial in range(40):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        # coarse values so that exact ties are common
        z = (rng.integers(-3, 4, size=(3, E)) * 0.25).astype(np.float32)
        ids = oracle.select_topk(z, k)
        for t in range(3):
            winners = _brute_topk(z[t].tolist(), k)
            assert len(winners) == 1
            assert ids[t].tolist() == winners[0]


def test_duplicate_router_rows_pick_lower_index():
    rng = np.random.default_rng(13)
    H, E = 256, 6
    wr = _bf16(rng.standard_normal((E, H)) * 0.02)
    wr[4] = wr[1]                     # experts 1 and 4 have identical logits
    wr[5] = wr[1]
    x = _bf16(rng.standard_normal((16, H)))
    z = oracle.router_logits(x, wr)
    assert np.array_equal(z[:, 1], z[:, 4])
    ids = oracle.select_topk(z, 2)
    for t in range(16):
        s = set(ids[t].tolist())
        if 4 in s:
            assert 1 in s
        if 5 in s:
            assert 1 in s and 4 in s
        assert ids[t].tolist() == sorted(s)


def test_weights_softmax_properties():
    rng = np.random.default_rng(14)
    z = rng.standard_normal((50, 12)).astype(np.float32) * 3
    k = 4
    ids = oracle.select_topk(z, k)
    w = oracle.gate_weights(z, ids)
    assert w.dtype == np.float32
    assert np.all(w > 0)
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1) <= 1e-6)
    # every selected logit is >= every unselected one
    for t in range(50):
        sel = z[t, ids[t]]
        rest = np.delete(z[t], ids[t])
        assert sel.min() >= rest.max()
        # weights are ordered like the logits, and match a scalar math.exp loop
        m = max(float(v) for v in sel)
        ex = [math.exp(float(v) - m) for v in sel]
        ref = [e / sum(ex) for e in ex]
        assert np.allclose(w[t], ref, rtol=0, atol=1e-7)


def test_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(15)
    z = rng.standard_normal((4, 6)).astype(np.float32)
    ids = oracle.select_topk(z, 6)
    assert np.array_equal(ids, np.tile(np.arange(6), (4, 1)))
    w = oracle.gate_weights(z, ids)
    for t in range(4):
        ex = [math.exp(float(v)) for v in z[t]]
        assert np.allclose(w[t], [e / sum(ex) for e in ex], rtol=0, atol=1e-7)


def test_permutation_against_sorted():
    rng = np.random.default_rng(16)
    T, E, k = 37, 9, 3
    ids = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    offsets, sorted_routes, route_pos = oracle.permutation(ids, E)
    routes = [(int(ids[t, j]), t, t * k + j) for t in range(T) for j in range(k)]
    expect = [r for (_, _, r) in sorted(routes)]
    assert sorted_routes.tolist() == expect
    counts = np.bincount(ids.reshape(-1), minlength=E)
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(route_pos[sorted_routes], np.arange(T * k))
    for e in range(E):
        seg = sorted_routes[offsets[e]:offsets[e + 1]]
        assert np.all(ids.reshape(-1)[seg] == e)
        assert np.all(np.diff(seg) > 0)
