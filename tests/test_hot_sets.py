"""The stored hot-expert table of the mixed-precision workloads equals routes
counted with the oracle (CPU only).

"Dynamic Expert Quantization for Scalable Mixture-of-Experts Inference"
(abstract): the experts kept at higher precision are the most used ones, with
usage taken from the routing.  inputs/hot_sets.json (written by
tests/golden/make_hot_sets.py) ranks each workload's experts by routes counted
over its full token set; the generator's tier table follows that ranking.
"""

import numpy as np
import pytest

import inputs
import oracle


@pytest.mark.parametrize("cid", [3, 4])
def test_hot_table_matches_oracle_route_counts(cid):
    cfg = inputs.get_config(cid)
    T = cfg.max_tokens
    x = inputs.gen_tokens(cfg, T)
    r = oracle.route(x, inputs.gen_router(cfg), inputs.gen_bias(cfg), cfg.top_k)
    counts = np.bincount(r["ids"].ravel(), minlength=cfg.n_experts)
    order = inputs.hot_order(cfg)
    assert sorted(order.tolist()) == list(range(cfg.n_experts))
    # descending counts, ties in increasing expert id
    c = counts[order]
    assert np.all(c[:-1] >= c[1:])
    for a, b in zip(order[:-1], order[1:]):
        if counts[a] == counts[b]:
            assert a < b
    tiers = inputs.gen_tiers(cfg)
    assert np.all(tiers[order[:cfg.n_bf16]] == inputs.TIER_BF16)
    assert np.all(tiers[order[cfg.n_bf16:cfg.n_bf16 + cfg.n_int8]] == inputs.TIER_INT8)
    assert np.all(tiers[order[cfg.n_bf16 + cfg.n_int8:]] == inputs.TIER_INT4)
    # every bf16 expert is routed at least as often as every int8 one, and so on
    if cfg.n_bf16:
        assert counts[tiers == 0].min() >= counts[tiers == 1].max()
    assert counts[tiers == 1].min() >= counts[tiers == 2].max()
