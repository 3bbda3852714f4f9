"""GPU routing vs the oracle: logits, ids, offsets, permutation bit-exact;
weights within 1e-6 (ExactMoE section 3.1 router and TopK; section 3.4 grouping)."""

import dataclasses

import numpy as np
import pytest

import inputs
import oracle
from tests._harness import Setup, log, to_dev

pytestmark = pytest.mark.gpu


def _check_route(st: Setup, layer=None):
    import torch
    log(f"route cfg{st.cfg.cid} T={st.T} E={st.E} k={st.k}")
    if layer is None:
        layer = st.gpu_layer(experts=[0])
    x, wr, b = st.dev_inputs()
    got = {k: v.cpu().numpy() for k, v in layer.route(x, wr, b).items()}
    torch.cuda.synchronize()
    ref = oracle.route(st.x, st.wr, st.bias, st.k)
    assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32)), \
        "logits differ"
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.max(np.abs(got["weights"] - ref["weights"])) <= 1e-6
    assert np.all(np.abs(got["weights"].astype(np.float64).sum(1) - 1) <= 1e-6)
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["sorted_routes"], ref["sorted_routes"])
    assert np.array_equal(got["route_pos"], ref["route_pos"])
    return layer


@pytest.mark.parametrize("cid,T", [(1, 64), (2, 32), (3, 512), (4, 1), (4, 32), (4, 256),
                                   (4, 4096), (5, 8192), (1, 1), (1, 37), (2, 5),
                                   # multi-block grouping (T > 1024): ragged last block,
                                   # a one-token last block
                                   (4, 1300), (4, 1025), (4, 2000)])
def test_route_bitexact(cid, T):
    _check_route(Setup(cid, T=T))


def test_route_exact_ties_lower_index():
    """Duplicate router rows give exactly equal logits; the lower id must win."""
    st = Setup(1, T=64)
    wr = st.wr.copy()
    wr[5] = wr[2]
    wr[7] = wr[2]
    wr[6] = wr[1]
    st.wr = wr
    _check_route(st)


def test_route_k_equals_e():
    cfg = inputs.get_config(1)
    import dataclasses
    c = dataclasses.replace(cfg, top_k=8, cid=1)
    st = Setup(1, T=16, cfg=c)
    _check_route(st)


def test_route_large_bias_forces_experts():
    st = Setup(2, T=32, bias=None)
    b = np.zeros(st.E, np.float32)
    b[[3, 77, 100, 101, 5, 9, 64, 127]] = 1000.0
    st.bias = b
    _check_route(st)


def _route_np(layer, st, want_logits):
    import torch
    x, wr, b = st.dev_inputs()
    got = {k: v.cpu().numpy() for k, v in layer.route(x, wr, b, want_logits=want_logits).items()}
    torch.cuda.synchronize()
    return got


def _tie_rows(st):
    wr = st.wr.copy()
    wr[5] = wr[2]
    wr[7] = wr[2]
    wr[6] = wr[1]
    st.wr = wr


def _big_bias(st):
    b = np.zeros(st.E, np.float32)
    b[np.arange(st.k) * (st.E // st.k)] = 1000.0
    st.bias = b


def _small_cfg(E, H, k, max_tokens=64):
    return dataclasses.replace(inputs.get_config(1), hidden=H, n_experts=E, top_k=k,
                               max_tokens=max_tokens)


@pytest.mark.parametrize("cid,T,mutate,shape", [
    (6, 32, None, None), (6, 1, None, None), (6, 63, None, None), (6, 17, _big_bias, None),
    (5, 7, None, None), (5, 64, None, None), (1, 64, _tie_rows, None), (1, 37, None, None),
    (1, 1, _tie_rows, None), (1, 64, None, (128, 1024, 8)), (1, 33, _big_bias, (128, 1024, 8)),
    (1, 20, None, (100, 768, 6)), (1, 64, None, (33, 2048, 4)), (1, 5, None, (32, 4096, 3))])
def test_small_router_matches_canonical(cid, T, mutate, shape):
    """Few tokens, no logits output, router weights up to 256 KiB: one block
    per token computes the logits in the canonical order and takes the top k
    on chip.  Same routing bit for bit as the logits + top-k kernels (ids,
    weights, offsets, permutation) and the oracle's: E = 8, 32, 33, 64, 100,
    128 (each expert-per-half-wave and expert-per-lane bound, full and
    ragged); one token; exact ties; forced experts."""
    st = Setup(cid, T=T) if shape is None else Setup(cid, T=T, cfg=_small_cfg(*shape))
    if mutate is not None:
        mutate(st)
    layer = st.gpu_layer(experts=[0])
    log(f"small route cfg{cid} T={T} E={st.E} k={st.k}")
    fast = _route_np(layer, st, False)
    canon = _route_np(layer, st, True)
    for key in ("ids", "offsets", "sorted_routes", "route_pos"):
        assert np.array_equal(fast[key], canon[key]), key
    assert np.array_equal(fast["weights"].view(np.uint32), canon["weights"].view(np.uint32))
    ref = oracle.route(st.x, st.wr, st.bias, st.k)
    assert np.array_equal(fast["ids"], ref["ids"])
    assert np.max(np.abs(fast["weights"] - ref["weights"])) <= 1e-6


@pytest.mark.parametrize("T", [64, 3, 200])
def test_route_1024_experts_top16(T):
    """The largest expert count and top-k the library takes (1024 experts,
    top-16, 512 KiB of router weights): the top-k kernel holds 16 entries per
    lane.  Routing bit-exact against the oracle."""
    _check_route(Setup(1, T=T, cfg=_small_cfg(1024, 256, 16, max_tokens=256)))


def _mfma_layer(st):
    from mixed_precision_moe_amd import ROUTER_MFMA
    layer = st.gpu_layer(experts=[0])
    layer.set_router_mode(ROUTER_MFMA)
    return layer


@pytest.mark.parametrize("cid,T", [(3, 512), (4, 4096), (4, 1025), (6, 512), (4, 256),
                                   (1, 37), (2, 1), (5, 300), (4, 33)])
def test_certified_router_matches_canonical(cid, T):
    """Without logits output, the MFMA router (approximate logits, error-bound
    candidates, canonical recompute) gives the canonical routing bit for bit
    (ids, weights, offsets, permutation), and the oracle's: ragged token
    tiles, one token, E below one 64-expert tile (E = 8, 32)."""
    st = Setup(cid, T=T)
    layer = _mfma_layer(st)
    log(f"MFMA route cfg{cid} T={T} E={st.E} k={st.k}")
    fast = _route_np(layer, st, False)
    canon = _route_np(layer, st, True)
    for key in ("ids", "offsets", "sorted_routes", "route_pos"):
        assert np.array_equal(fast[key], canon[key]), key
    assert np.array_equal(fast["weights"].view(np.uint32), canon["weights"].view(np.uint32))
    ref = oracle.route(st.x, st.wr, st.bias, st.k)
    assert np.array_equal(fast["ids"], ref["ids"])
    assert np.max(np.abs(fast["weights"] - ref["weights"])) <= 1e-6


def test_certified_router_exact_ties_among_candidates():
    """The router rows (and biases) come in groups of four exact copies, so the
    top-k boundary of every token (k = 10) cuts through a group of equal
    logits: the whole group is among the candidates and the canonical tie
    rule (lower id first) decides inside the MFMA router's selection."""
    st = Setup(4, T=512)
    B = st.E // 4
    wr = st.wr.copy()
    for g in range(1, 4):
        wr[g * B:(g + 1) * B] = wr[:B]
    st.wr = wr
    if st.bias is not None:
        b = st.bias.copy()
        for g in range(1, 4):
            b[g * B:(g + 1) * B] = b[:B]
        st.bias = b
    assert st.k % 4 != 0
    layer = _mfma_layer(st)
    fast = _route_np(layer, st, False)
    canon = _route_np(layer, st, True)
    for key in ("ids", "offsets", "sorted_routes", "route_pos"):
        assert np.array_equal(fast[key], canon[key]), key
    assert np.array_equal(fast["weights"].view(np.uint32), canon["weights"].view(np.uint32))
    ref = oracle.route(st.x, st.wr, st.bias, st.k)
    assert np.array_equal(fast["ids"], ref["ids"])
    # whole groups first, then the lowest copies of the cut group
    q, r = divmod(st.k, 4)
    want = np.array([q + (g < r) for g in range(4)])
    counts = np.stack([np.sum(fast["ids"] // B == g, axis=1) for g in range(4)], axis=1)
    assert np.all(counts == want)


def test_certified_router_full_ties():
    """Every other token is zero and there is no bias: all of its logits are
    exactly 0, every expert stays a candidate, and the canonical recompute of
    all of them routes the token to the k lowest ids with equal weights; the
    other tokens have a few candidates each, in the same call."""
    st = Setup(4, T=384, bias=None)
    x = st.x.copy()
    x[::2] = 0
    st.x = x
    layer = _mfma_layer(st)
    fast = _route_np(layer, st, False)
    canon = _route_np(layer, st, True)
    for key in ("ids", "offsets", "sorted_routes", "route_pos"):
        assert np.array_equal(fast[key], canon[key]), key
    assert np.array_equal(fast["weights"].view(np.uint32), canon["weights"].view(np.uint32))
    ref = oracle.route(st.x, st.wr, st.bias, st.k)
    assert np.array_equal(fast["ids"], ref["ids"])
    assert np.max(np.abs(fast["weights"] - ref["weights"])) <= 1e-6
    assert np.all(fast["ids"][::2] == np.arange(st.k)[None, :])
    assert np.max(np.abs(fast["weights"][::2] - 1.0 / st.k)) <= 1e-6


def test_router_mode_workspace_and_errors():
    """The MFMA router needs its partial logits in the workspace: the size
    follows the mode, and a bad mode is refused."""
    from mixed_precision_moe_amd import ROUTER_AUTO, ROUTER_CANONICAL, ROUTER_MFMA, MoeError
    st = Setup(3, T=64)
    layer = st.gpu_layer(experts=[0])
    layer.set_router_mode(ROUTER_CANONICAL)
    small = layer.workspace_size(512)
    layer.set_router_mode(ROUTER_MFMA)
    big = layer.workspace_size(512)
    assert big > small
    layer.set_router_mode(ROUTER_AUTO)
    with pytest.raises(MoeError):
        layer.set_router_mode(7)
