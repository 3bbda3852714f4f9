"""The benchmark's accounting, checked on the CPU.

bench.py turns kernel times into roofline fractions with algorithmic byte and
flop counts.  These tests pin those counts to things fixed elsewhere: the
packed size of each tier against the library's own moe_packed_size (and, for
int4, the memory equation of "Every Expert Counts: ExactMoE ...", section
3.2: n k / 2 code bytes plus one 16-bit scale per 128 weights); the byte and
flop sums against a hand count on a small routing; and the headline
workload's touched experts against the oracle's routing.
"""

import ctypes

import numpy as np
import pytest

import bench
import inputs
import oracle


def _lib_or_skip():
    from mixed_precision_moe_amd import _lib
    try:
        return _lib.load()
    except ImportError as e:   # the library is built by __graft_entry__.build()
        pytest.skip(str(e))


@pytest.mark.parametrize("tier", [0, 1, 2])
@pytest.mark.parametrize("n,k", [(64, 128), (1536, 2048), (2048, 768), (28672, 4096)])
def test_packed_bytes_match_library_and_memory_equation(tier, n, k):
    lib = _lib_or_skip()
    lib.moe_packed_size.restype = ctypes.c_size_t
    lib.moe_packed_size.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    got = bench.packed_bytes(tier, n, k)
    # the library rounds each blob up to 256 bytes; the payload is the same
    assert lib.moe_packed_size(tier, n, k) == (got + 255) // 256 * 256
    per_param = {2: 0.5 + 2 / 128, 1: 1.0 + 2 / k, 0: 2.0}[tier]
    assert got == pytest.approx(n * k * per_param, rel=0, abs=0.5)


def test_algorithmic_counts_by_hand():
    """The tiny layer (8 experts), two of them touched, one int8 and one
    int4; T = 3."""
    cfg = inputs.get_config(1)
    H, I, k, E, T = cfg.hidden, cfg.inter, cfg.top_k, cfg.n_experts, 3
    tiers = np.full(E, 2, np.int32)
    tiers[5] = 1
    ids = np.array([[1, 5], [1, 5], [1, 5]], np.int32)
    a = bench.algorithmic(cfg, tiers, ids, T)
    w13 = (2 * I * H // 2 + 2 * I * (H // 128) * 2) + (2 * I * H + 2 * 2 * I)
    w2 = (H * I // 2 + H * (I // 128) * 2) + (H * I + 2 * H)
    assert a["touched"] == 2
    assert a["bytes13"] == w13 + 2 * T * H + 2 * T * k * I
    assert a["bytes2"] == w2 + 2 * T * k * I + 4 * T * k * H
    assert a["flops13"] == 2.0 * T * k * H * 2 * I
    assert a["flops2"] == 2.0 * T * k * I * H
    assert a["bytes_layer"] == w13 + w2 + 4 * T * H + 2 * E * H
    assert a["flops_layer"] == a["flops13"] + a["flops2"]


def test_headline_workload_counts_from_oracle_routing():
    """The Qwen3-30B-shaped decode batch (32 tokens, top-8 of 128 int4
    experts): the oracle's routing touches 115 experts, and the layer's
    algorithmic bytes are their packed weights (2,433,024 bytes per expert)
    plus x, y and the router."""
    cfg = inputs.get_config(2)
    x, wr = inputs.gen_tokens(cfg), inputs.gen_router(cfg)
    r = oracle.route(x, wr, inputs.gen_bias(cfg), cfg.top_k)
    tiers = inputs.gen_tiers(cfg)
    a = bench.algorithmic(cfg, tiers, r["ids"], cfg.default_tokens)
    T, H, E = cfg.default_tokens, cfg.hidden, cfg.n_experts
    assert a["touched"] == len(np.unique(r["ids"])) == 115
    assert a["bytes_layer"] == 115 * 2_433_024 + 4 * T * H + 2 * E * H
    # the gate/up kernel's algorithmic bytes per launch, as the bench line reports them
    assert a["bytes13"] == 187_056_128
