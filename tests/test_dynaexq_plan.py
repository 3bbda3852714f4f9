"""DynaExq's tier plan: the n most used experts that fit a byte budget take the
high tier (CPU only).

The oracle's rule is pinned by brute force over every subset of a small
expert set (the chosen set is the largest feasible one made of the hottest
experts, ties to the lower id); the library's host planner must give the same
tiers and count on random cases.
"""

import itertools
import os

import numpy as np
import pytest

import oracle
from mixed_precision_moe_amd import _lib

SIZES = [9437184, 4725760, 2433024]     # one Qwen3-30B-shaped expert per tier: bf16, int8, int4


def _brute(hot, sizes, budget, hi, lo):
    E = len(hot)
    rank = sorted(range(E), key=lambda e: (-hot[e], e))
    best = None
    for n in range(E + 1):
        for sub in itertools.combinations(range(E), n):
            cost = sum(sizes[hi] if e in sub else sizes[lo] for e in range(E))
            if cost > budget:
                continue
            # among feasible sets of the largest size, the hottest prefix
            if set(sub) == set(rank[:n]):
                best = (n, sub)
    return best


@pytest.mark.parametrize("seed", range(6))
def test_plan_rule_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    E = 7
    hot = rng.integers(0, 5, size=E).astype(float).tolist()     # many ties
    lo = SIZES[2] * E
    budget = lo + int(rng.integers(0, 5)) * (SIZES[0] - SIZES[2]) + int(rng.integers(0, 1000))
    tiers, n = oracle.plan_tiers(hot, SIZES, budget, 0, 2)
    nb, sub = _brute(hot, SIZES, budget, 0, 2)
    assert n == nb
    assert sorted(e for e in range(E) if tiers[e] == 0) == sorted(sub)


def test_plan_rule_edges():
    hot = [3.0, 1.0, 3.0, 0.0]
    # exact fit for two promotions; the tie between experts 0 and 2 keeps both
    budget = 2 * SIZES[0] + 2 * SIZES[2]
    tiers, n = oracle.plan_tiers(hot, SIZES, budget, 0, 2)
    assert n == 2 and tiers == [0, 2, 0, 2]
    tiers, n = oracle.plan_tiers(hot, SIZES, budget - 1, 0, 2)
    assert n == 1 and tiers == [0, 2, 2, 2]      # tie -> lower id
    tiers, n = oracle.plan_tiers(hot, SIZES, 10 ** 12, 1, 2)
    assert n == 4 and tiers == [1, 1, 1, 1]
    with pytest.raises(ValueError):
        oracle.plan_tiers(hot, SIZES, 4 * SIZES[2] - 1, 0, 2)


pytestmark_lib = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmoe.so not built")


@pytestmark_lib
@pytest.mark.parametrize("seed", range(8))
def test_library_planner_matches_oracle(seed):
    from mixed_precision_moe_amd import plan_tiers
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 300))
    hot = rng.integers(0, 50, size=E).astype(np.float32).tolist()
    hi, lo = [(0, 2), (1, 2), (0, 1)][seed % 3]
    base = E * SIZES[lo]
    budget = base + int(rng.integers(0, E + 2)) * (SIZES[hi] - SIZES[lo]) + int(rng.integers(0, 10 ** 6))
    got = plan_tiers(hot, SIZES, budget, hi, lo)
    want = oracle.plan_tiers(hot, SIZES, budget, hi, lo)
    assert got[1] == want[1] and got[0] == want[0]


@pytestmark_lib
def test_library_planner_errors():
    from mixed_precision_moe_amd import MoeError, plan_tiers
    with pytest.raises(MoeError) as ei:
        plan_tiers([1.0, 2.0], SIZES, 2 * SIZES[2] - 1, 0, 2)
    assert ei.value.status == _lib.MOE_ENOSPC
    with pytest.raises(MoeError) as ei:
        plan_tiers([1.0, float("nan")], SIZES, 10 ** 9, 0, 2)
    assert ei.value.status == _lib.MOE_EINVAL
