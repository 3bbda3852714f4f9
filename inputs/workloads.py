"""Workload table and seeded generators for synthetic MoE layers.

Every array is drawn from numpy's PCG64 generator seeded with a tuple
(seed, config id, stream, index), so any single expert can be regenerated on
its own without drawing the others.  Values are drawn as float32 and stored
as bf16 bit patterns (uint16) rounded to nearest-even; that rounding is the
storage format of the inputs, not part of the layer.

Shapes follow the layer geometries the MoE pages discuss: a tiny layer, a
Qwen3-30B-A3B-shaped layer (decode and a skewed mixed-precision batch), a
Qwen3-80B-shaped layer with many small experts, and a Mixtral-shaped layer
for prefill.  The mixed-precision hot sets follow the DynaExq idea (Dynamic
Expert Quantization, abstract): the most used experts are held at higher
precision, the rest at an int4 fallback.  Usage is the routes counted over
the workload's full token set; the ranking is a stored table
(hot_sets.json beside this file, written by tests/golden/make_hot_sets.py),
so this module itself does no routing.
"""

from __future__ import annotations

import dataclasses
import functools
import json
import os
from typing import Dict, Optional, Tuple

import numpy as np

HOT_SETS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hot_sets.json")

TIER_BF16 = 0
TIER_INT8 = 1
TIER_INT4 = 2

# stream ids inside one config's seed tuple
_S_TOKENS, _S_ROUTER, _S_BIAS, _S_EXPERT = 0, 1, 2, 4

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    cid: int
    name: str
    hidden: int          # H
    n_experts: int       # E
    top_k: int           # k
    inter: int           # I (expert intermediate size)
    tokens: Tuple[int, ...]   # token counts exercised (first is the default)
    max_tokens: int      # rows of x that are drawn; smaller T use the first T rows
    zipf_bias: Optional[float] = None   # s of the Zipf router bias, if any
    n_bf16: int = 0      # hottest experts kept in bf16
    n_int8: int = 0      # next hottest kept in int8 per-channel
    seed: int = 0

    @property
    def default_tokens(self) -> int:
        return self.tokens[0]

    def describe(self, T: Optional[int] = None) -> str:
        T = self.default_tokens if T is None else T
        if self.n_bf16 or self.n_int8:
            prec = f"{self.n_bf16} bf16 / {self.n_int8} int8 / " \
                   f"{self.n_experts - self.n_bf16 - self.n_int8} int4-g128"
        else:
            prec = "all int4-g128"
        bias = f", Zipf(s={self.zipf_bias}) router bias" if self.zipf_bias else ""
        return (f"{self.name}: H{self.hidden} E{self.n_experts} top{self.top_k} "
                f"I{self.inter} SwiGLU, {prec}{bias}, T={T}")


CONFIGS: Dict[int, LayerConfig] = {
    1: LayerConfig(1, "tiny MoE layer", 256, 8, 2, 512, (64,), 64),
    2: LayerConfig(2, "Qwen3-30B-A3B-shaped MoE layer, decode", 2048, 128, 8, 768,
                   (32,), 32),
    3: LayerConfig(3, "Qwen3-30B-A3B-shaped MoE layer, mixed precision", 2048, 128, 8,
                   768, (512,), 512, zipf_bias=1.1, n_bf16=16, n_int8=32),
    4: LayerConfig(4, "Qwen3-80B-shaped MoE layer", 2048, 512, 10, 512,
                   (32, 1, 256, 4096), 4096, n_int8=64),
    5: LayerConfig(5, "Mixtral-shaped MoE layer, prefill", 4096, 8, 2, 14336,
                   (8192,), 8192),
    # the second model family the ExactMoE page measures (OLMoE: 64 experts,
    # top-8); decode batch of 32 and a 512-token prefill chunk
    6: LayerConfig(6, "OLMoE-shaped MoE layer", 2048, 64, 8, 1024, (32, 512), 512),
}


def get_config(cid: int) -> LayerConfig:
    return CONFIGS[int(cid)]


def _rng(cfg: LayerConfig, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, cfg.cid, stream, index])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def gen_tokens(cfg: LayerConfig, T: Optional[int] = None) -> np.ndarray:
    """x: [T, H] bf16 bits, N(0, 1).  Smaller T take the first T rows."""
    T = cfg.default_tokens if T is None else int(T)
    if T > cfg.max_tokens:
        raise ValueError(f"T={T} exceeds the {cfg.max_tokens} rows drawn for config {cfg.cid}")
    x = _normal_bf16(_rng(cfg, _S_TOKENS), (cfg.max_tokens, cfg.hidden), 1.0)
    return np.ascontiguousarray(x[:T])


def gen_router(cfg: LayerConfig) -> np.ndarray:
    """Router weight as the library takes it: [E, H] bf16 bits, N(0, 0.02).

    The draw is made as an [H, E] matrix (the orientation in which the tiny
    config is stated) and transposed.
    """
    w_he = _normal_bf16(_rng(cfg, _S_ROUTER), (cfg.hidden, cfg.n_experts), WEIGHT_STD)
    return np.ascontiguousarray(w_he.T)


def _popularity_rank(cfg: LayerConfig, stream: int) -> np.ndarray:
    """rank[e] in 1..E: a seeded permutation, 1 = most popular."""
    perm = _rng(cfg, stream).permutation(cfg.n_experts)
    return (perm + 1).astype(np.int64)


def gen_bias(cfg: LayerConfig) -> Optional[np.ndarray]:
    """Router bias [E] float32, or None.

    For a Zipf(s) popularity law p_e ~ rank_e^(-s), the bias is the log
    popularity, b_e = -s * ln(rank_e), so exp(z + b) weights experts by that law.
    """
    if not cfg.zipf_bias:
        return None
    rank = _popularity_rank(cfg, _S_BIAS)
    b = -cfg.zipf_bias * np.log(rank.astype(np.float64))
    return b.astype(np.float32)


@functools.lru_cache(maxsize=None)
def _hot_table() -> dict:
    with open(HOT_SETS) as f:
        return json.load(f)


def hot_order(cfg: LayerConfig) -> np.ndarray:
    """Experts of a mixed-precision workload, most routed first (routes counted
    over its full token set, ties to the lower id), from the stored table."""
    entry = _hot_table().get(str(cfg.cid))
    if entry is None or len(entry["order"]) != cfg.n_experts:
        raise ValueError(f"no hot-expert table for config {cfg.cid} "
                         f"(run tests/golden/make_hot_sets.py)")
    return np.asarray(entry["order"], dtype=np.int64)


def gen_tiers(cfg: LayerConfig) -> np.ndarray:
    """Per-expert precision tier [E] int32 (0 bf16, 1 int8, 2 int4).

    The n_bf16 most routed experts are bf16, the next n_int8 int8 per-channel,
    the rest int4 group-128 (hot_order).
    """
    tiers = np.full(cfg.n_experts, TIER_INT4, dtype=np.int32)
    if not (cfg.n_bf16 or cfg.n_int8):
        return tiers
    order = hot_order(cfg)
    tiers[order[:cfg.n_bf16]] = TIER_BF16
    tiers[order[cfg.n_bf16:cfg.n_bf16 + cfg.n_int8]] = TIER_INT8
    return tiers


def gen_expert(cfg: LayerConfig, e: int):
    """Master weights of expert e as bf16 bits, each N(0, 0.02).

    Returns (w_gate [I, H], w_up [I, H], w_down [H, I]), PyTorch Linear
    orientation ([out, in]).
    """
    rng = _rng(cfg, _S_EXPERT, int(e))
    H, I = cfg.hidden, cfg.inter
    w_gate = _normal_bf16(rng, (I, H), WEIGHT_STD)
    w_up = _normal_bf16(rng, (I, H), WEIGHT_STD)
    w_down = _normal_bf16(rng, (H, I), WEIGHT_STD)
    return w_gate, w_up, w_down


def expected_touched(cfg: LayerConfig, T: int) -> float:
    """Expected distinct experts touched by T uniform tokens (no bias)."""
    E, k = cfg.n_experts, cfg.top_k
    return E * (1.0 - (1.0 - k / E) ** T)
