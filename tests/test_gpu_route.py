"""GPU routing vs the oracle: logits, ids, offsets, permutation bit-exact;
weights within 1e-6 (ExactMoE section 3.1 router and TopK; section 3.4 grouping)."""

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
