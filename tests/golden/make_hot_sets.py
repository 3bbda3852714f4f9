"""Write inputs/hot_sets.json: the hot-expert order of the mixed-precision
workloads, from counted routes (oracle only).

"Dynamic Expert Quantization for Scalable Mixture-of-Experts Inference"
(abstract) keeps the most used experts of a layer at higher precision, with
usage estimated from the layer's routing.  Reading taken for the synthetic
workloads: route every token of the workload's full token set with the
oracle (router logits in the canonical fp32 order, top-k with ties to the
lower id), count the (token, slot) assignments per expert, and rank experts
by count, descending, ties to the lower id.  The workload generator then
gives the first n_bf16 experts of that order the bf16 tier and the next
n_int8 the int8 tier (the Qwen3-30B-A3B-shaped layer: 512 tokens with its
Zipf router bias; the Qwen3-80B-shaped layer: all 4096 tokens, one table for
every token count of its sweep).

    python tests/golden/make_hot_sets.py

The table depends only on the seeded tokens and router weights, not on the
tiers, so there is no circularity.  tests/test_hot_sets.py recomputes it.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import inputs  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(ROOT, "inputs", "hot_sets.json")


def hot_order(cid: int):
    """(route counts per expert, experts ranked by count desc, id asc)."""
    cfg = inputs.get_config(cid)
    T = cfg.max_tokens
    x = inputs.gen_tokens(cfg, T)
    r = oracle.route(x, inputs.gen_router(cfg), inputs.gen_bias(cfg), cfg.top_k)
    counts = np.bincount(r["ids"].ravel(), minlength=cfg.n_experts)
    order = sorted(range(cfg.n_experts), key=lambda e: (-int(counts[e]), e))
    return T, counts, order


def main():
    table = {"about": "experts of each mixed-precision workload ranked by routes counted "
                      "over its full token set (oracle routing); written by "
                      "tests/golden/make_hot_sets.py"}
    for cid in sorted(inputs.CONFIGS):
        cfg = inputs.get_config(cid)
        if not (cfg.n_bf16 or cfg.n_int8):
            continue
        T, counts, order = hot_order(cid)
        table[str(cid)] = {"tokens": T, "order": [int(e) for e in order],
                           "counts": [int(c) for c in counts]}
        print(f"config {cid}: {T} tokens, hottest {order[:8]} with "
              f"{[int(counts[e]) for e in order[:8]]} routes", flush=True)
    with open(OUT, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
