"""Oracle for the quantized MoE FFN layer (numpy; CPU; test infrastructure only).

Sources (the web pages the method is taken from):
  [ExactMoE]  "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference"
              -- §3.1 (router equation, dequantized values define the operations),
              §3.2 (symmetric group-128 quantizer; memory equation),
              §3.3 (packed weights with FP16 scales), §3.4 (grouped execution,
              router weights kept across waves, output = sum of disjoint parts).
  [DynaExq]   "Dynamic Expert Quantization for Scalable Mixture-of-Experts
              Inference" -- abstract (hot experts at higher precision, low
              precision fallback for the rest).
  [MxMoE]     MxMoE abstract (mixed-precision GroupGEMM: GEMMs of different
              precisions executed together).

Where the pages are silent the reading taken is stated at the function that
depends on it.  No function here has a GPU counterpart it calls or imports.

Parity pins for every function live in tests/test_oracle_*.py (closed forms,
hand-worked groups, brute force on tiny inputs, textbook reductions).
"""

from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Optional, Sequence

import numpy as np

TIER_BF16, TIER_INT8, TIER_INT4 = 0, 1, 2
GROUP = 128                 # [ExactMoE] §3.2: group size of the W4 quantizer
INT4_QMAX, INT4_QMIN = 7, -8
INT8_QMAX, INT8_QMIN = 127, -128


# --------------------------------------------------------------------------- #
# number formats                                                              #
# --------------------------------------------------------------------------- #

def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact: bf16 is the top half of fp32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Written as integer arithmetic on the fp32 bit pattern: drop the low 16 bits
    after adding half an ulp of the kept part, biased by the kept LSB so exact
    halves go to the even neighbour.  Finite inputs only.
    """
    a = np.asarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite value in bf16 rounding")
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    out = (bits + 0x7FFF + lsb) >> 16
    return out.astype(np.uint16)


def _fp16(a) -> np.ndarray:
    """float32 -> IEEE binary16, round to nearest even (numpy's conversion)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------- #
# quantizers ([ExactMoE] §3.2; int8 tier by analogy, [DynaExq] abstract)      #
# --------------------------------------------------------------------------- #

def quantize_int4_g128(w_bf16: np.ndarray):
    """Symmetric int4 quantization with one scale per (row, 128-column group).

    [ExactMoE] §3.2, quantizer equation: s = max|W| over the group / 7,
    q = clip(round(W / s), -8, 7).  Readings where the page is silent:
      * groups are 128 consecutive entries along the input dimension of each
        output row (the row of a PyTorch Linear weight);
      * the scale is stored as FP16 ([ExactMoE] §3.3 and §6 name FP16 scales;
        the memory equation counts 16 bits per group).  It is computed as the
        float32 quotient max/7, rounded to fp16 (nearest even), and the codes
        are derived from that stored scale;
      * round() is round-half-to-even of the float32 quotient w/s;
      * an all-zero group has s = 0 and all codes 0;
      * a scale that overflows fp16 (or a non-finite weight) is an error.
    Returns q int8 [N, K] and s float16 [N, K/128].
    """
    w = bf16_bits_to_f32(w_bf16)
    if w.ndim != 2 or w.shape[1] % GROUP:
        raise ValueError("int4 quantization needs a 2-D weight with K % 128 == 0")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    N, K = w.shape
    wg = w.reshape(N, K // GROUP, GROUP)
    m = np.max(np.abs(wg), axis=2)                                  # exact
    s16 = _fp16(m / np.float32(INT4_QMAX))                          # fp32 divide, fp16 RNE
    if not np.all(np.isfinite(s16)):
        raise ValueError("fp16 scale overflow")
    s32 = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s32 != 0, wg / np.where(s32 != 0, s32, 1), 0).astype(np.float32)
    q = np.clip(np.rint(ratio), INT4_QMIN, INT4_QMAX).astype(np.int8)
    return q.reshape(N, K), s16


def quantize_int8_per_channel(w_bf16: np.ndarray):
    """Symmetric int8 quantization with one scale per output row.

    The int8 tier is not specified on the pages beyond being a higher
    precision for hot experts ([DynaExq] abstract; [MxMoE] abstract).  Reading:
    the int4 rule of [ExactMoE] §3.2 with the group widened to the whole row and
    the range widened to int8: s = fp16(max|w_row| / 127), q = clip(rint(w/s),
    -128, 127).  Returns q int8 [N, K] and s float16 [N].
    """
    w = bf16_bits_to_f32(w_bf16)
    if w.ndim != 2:
        raise ValueError("int8 quantization needs a 2-D weight")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    m = np.max(np.abs(w), axis=1)
    s16 = _fp16(m / np.float32(INT8_QMAX))
    if not np.all(np.isfinite(s16)):
        raise ValueError("fp16 scale overflow")
    s32 = s16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s32 != 0, w / np.where(s32 != 0, s32, 1), 0).astype(np.float32)
    q = np.clip(np.rint(ratio), INT8_QMIN, INT8_QMAX).astype(np.int8)
    return q, s16


def dequantize(tier: int, q, s, w_bf16=None) -> np.ndarray:
    """Dequantized weight in float64: W_hat = q * s (exact in float64).

    [ExactMoE] §3.1: the dequantized values define the operation; no rounding of
    W_hat to a 16-bit type is part of it.  bf16-tier experts use the master
    bf16 weight as is.
    """
    if tier == TIER_BF16:
        return bf16_bits_to_f32(w_bf16).astype(np.float64)
    q64 = np.asarray(q, dtype=np.float64)
    s64 = np.asarray(s, dtype=np.float64)
    if tier == TIER_INT4:
        N, K = q64.shape
        return (q64.reshape(N, K // GROUP, GROUP) * s64[:, :, None]).reshape(N, K)
    if tier == TIER_INT8:
        return q64 * s64[:, None]
    raise ValueError(f"bad tier {tier}")


def quantize_tier(tier: int, w_bf16: np.ndarray):
    """(q, s) for a quantized tier, (None, None) for bf16."""
    if tier == TIER_INT4:
        return quantize_int4_g128(w_bf16)
    if tier == TIER_INT8:
        return quantize_int8_per_channel(w_bf16)
    if tier == TIER_BF16:
        return None, None
    raise ValueError(f"bad tier {tier}")


# --------------------------------------------------------------------------- #
# routing ([ExactMoE] §3.1 router equation and TopK)                          #
# --------------------------------------------------------------------------- #

N_CHAINS = 32        # canonical logit order: 32 partial sums
CHAIN_WIDTH = 8      # ... each taking 8 consecutive terms per 256-wide slab
SLAB = N_CHAINS * CHAIN_WIDTH


def router_logits(x_bf16: np.ndarray, wr_bf16: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] * Wr[e, h] + b[e], in float32, canonical order.

    [ExactMoE] §3.1: z = W_r h with the router kept in BF16.  The page fixes
    neither the accumulation precision nor the order; because the top-k choice
    must be reproducible bit for bit, the reading is float32 in one fixed
    order:
      * chain j (0..31) starts at +0 and adds, in sequence, the products at
        h = 256*i + 8*j + r for slab i = 0, 1, ... (outer) and r = 0..7 (inner);
        each bf16*bf16 product is exact in float32, so every add rounds once;
      * the 32 chains are folded pairwise: for s = 16, 8, 4, 2, 1 chain j (< s)
        becomes chain j + chain j+s;
      * the bias (0 when absent) is added last.
    Needs H % 256 == 0.  Returns float32 [T, E].
    """
    x = bf16_bits_to_f32(x_bf16)
    w = bf16_bits_to_f32(wr_bf16)
    T, H = x.shape
    E, H2 = w.shape
    if H != H2 or H % SLAB:
        raise ValueError("router needs matching H with H % 256 == 0")
    chains = np.zeros((T, E, N_CHAINS), dtype=np.float32)
    j = np.arange(N_CHAINS)
    for i in range(H // SLAB):
        for r in range(CHAIN_WIDTH):
            cols = SLAB * i + CHAIN_WIDTH * j + r                 # [32]
            prod = x[:, None, cols] * w[None, :, cols]           # exact fp32 products
            chains += prod                                       # one fp32 rounding each
    s = N_CHAINS // 2
    while s >= 1:
        chains[:, :, :s] = chains[:, :, :s] + chains[:, :, s:2 * s]
        s //= 2
    z = chains[:, :, 0]
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    return (z + b[None, :]).astype(np.float32)


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """S_t = TopK(z_t, k) ([ExactMoE] §3.1), as expert ids ascending.

    Ties between equal logits go to the lower expert index (a stable sort of
    -z keeps index order among equals).  The selected set is stored in
    ascending expert order, so the position of an expert inside a token's k
    slots never depends on near-ties within the set.
    """
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.argsort(-z[t].astype(np.float64), kind="stable")
        ids[t] = np.sort(order[:k])
    return ids


def gate_weights(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Routing weights: softmax over the k selected logits, float64 -> float32.

    Reading (the pages name only TopK): the common top-k softmax, i.e. the full
    softmax renormalized over the selected set, which is the same thing.
    [ExactMoE] §3.4 keeps these weights across waves without renormalizing per
    wave, so they are computed once over the whole selected set.
    """
    zs = np.take_along_axis(z.astype(np.float64), ids.astype(np.int64), axis=1)
    m = zs.max(axis=1, keepdims=True)
    ex = np.exp(zs - m)
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def permutation(ids: np.ndarray, n_experts: int):
    """Group routes by expert ([ExactMoE] Fig. 1 and §3.4: tokens are grouped by
    selected expert before the grouped GEMMs).

    Route r = t*k + j is slot j of token t.  Reading: a stable grouping -- routes
    sorted by (expert, token), which for distinct experts within a token is a
    stable sort of the flat ids.  Returns
      offsets [E+1]   exclusive prefix sum of per-expert counts,
      sorted_routes   [T*k] route ids in grouped order,
      route_pos       [T*k] position of each route in that order (the inverse).
    """
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_routes = np.argsort(flat, kind="stable").astype(np.int32)
    route_pos = np.empty_like(sorted_routes)
    route_pos[sorted_routes] = np.arange(flat.size, dtype=np.int32)
    return offsets, sorted_routes, route_pos


def route(x_bf16, wr_bf16, bias, k):
    """Router logits, top-k ids, weights and the grouping permutation."""
    z = router_logits(x_bf16, wr_bf16, bias)
    ids = select_topk(z, k)
    w = gate_weights(z, ids)
    offsets, sorted_routes, route_pos = permutation(ids, wr_bf16.shape[0])
    return dict(logits=z, ids=ids, weights=w, offsets=offsets,
                sorted_routes=sorted_routes, route_pos=route_pos)


# --------------------------------------------------------------------------- #
# expert FFN and combine                                                      #
# --------------------------------------------------------------------------- #

def _silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def expert_ffn(x_rows: np.ndarray, wg_hat: np.ndarray, wu_hat: np.ndarray,
               wd_hat: np.ndarray) -> np.ndarray:
    """One expert on a block of token rows (float64 in, float64 out).

    [ExactMoE] §3.1 names the expert projections W_g, W_u and W_d; the gated
    form is SwiGLU: a = silu(W_g x) * (W_u x), y = W_d a.  W4A16 (the paper's
    title and §1) keeps activations in 16 bits, so the activation that feeds the
    down projection is rounded to bf16 (via float32, nearest even) before it.
    x_rows [m, H] (already bf16-exact), W_hat float64.  Returns [m, H].
    """
    g = x_rows @ wg_hat.T
    u = x_rows @ wu_hat.T
    a = _silu(g) * u
    a16 = bf16_bits_to_f32(f32_to_bf16_rne(a.astype(np.float32))).astype(np.float64)
    return a16 @ wd_hat.T


@dataclasses.dataclass
class OracleExpert:
    tier: int
    wg_hat: np.ndarray
    wu_hat: np.ndarray
    wd_hat: np.ndarray


def make_expert(tier: int, w_gate, w_up, w_down) -> OracleExpert:
    """Quantize (for int tiers) and dequantize one expert's three projections.

    The gate and up projections are quantized as one [2I, H] matrix
    (gate rows first); groups never straddle rows, so this equals quantizing
    each separately.
    """
    I = w_gate.shape[0]
    w13 = np.concatenate([w_gate, w_up], axis=0)
    q13, s13 = quantize_tier(tier, w13)
    q2, s2 = quantize_tier(tier, w_down)
    w13_hat = dequantize(tier, q13, s13, w13)
    w2_hat = dequantize(tier, q2, s2, w_down)
    return OracleExpert(tier, w13_hat[:I], w13_hat[I:], w2_hat)


def layer_forward(x_bf16: np.ndarray, routing: Dict[str, np.ndarray],
                  get_expert: Callable[[int], OracleExpert],
                  token_subset: Optional[Sequence[int]] = None) -> np.ndarray:
    """MoE layer output (float64 -> float32) from routing and dequantized experts.

    The output equation the pages refer to ("Equation 2" in [ExactMoE] §3.4) is
    not printed; reading: y_t = sum over e in S_t of w_{t,e} * FFN_e(x_t).  The
    sum runs over the token's slots in ascending expert order, in float64.
    [ExactMoE] §3.4 states that summing the contributions of disjoint expert
    subsets recovers this output; tests check that property.
    get_expert(e) is called once per expert the (sub)set of tokens selects.
    """
    x = bf16_bits_to_f32(x_bf16).astype(np.float64)
    ids, w = routing["ids"], routing["weights"].astype(np.float64)
    T, k = ids.shape
    toks = np.arange(T) if token_subset is None else np.asarray(token_subset)
    H = x.shape[1]
    contrib = np.zeros((len(toks), k, H), dtype=np.float64)
    for e in np.unique(ids[toks]):
        ex = get_expert(int(e))
        sel = np.nonzero(ids[toks] == e)          # (row in subset, slot)
        rows = x[toks[sel[0]]]
        contrib[sel[0], sel[1]] = expert_ffn(rows, ex.wg_hat, ex.wu_hat, ex.wd_hat)
        del ex
    out = np.zeros((len(toks), H), dtype=np.float64)
    for j in range(k):                            # slots are ascending by expert
        out += w[toks, j][:, None] * contrib[:, j]
    return out.astype(np.float32)


def wave_forward(x_bf16: np.ndarray, routing: Dict[str, np.ndarray],
                 get_expert: Callable[[int], OracleExpert], active) -> np.ndarray:
    """One wave of [ExactMoE] §3.4: the layer output restricted to the routes
    whose expert is in `active` (the experts mapped to a resident slot; every
    other expert maps to the inactive sentinel and contributes nothing).  The
    router weights are the full top-k softmax, not renormalized within the
    wave, so the waves of a partition of the experts sum to layer_forward.
    """
    x = bf16_bits_to_f32(x_bf16).astype(np.float64)
    ids, w = routing["ids"], routing["weights"].astype(np.float64)
    T, k = ids.shape
    H = x.shape[1]
    members = set(int(e) for e in active)
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):                            # slots ascending by expert
        for e in np.unique(ids[:, j]):
            if int(e) not in members:
                continue
            ex = get_expert(int(e))
            rows = np.nonzero(ids[:, j] == e)[0]
            out[rows] += w[rows, j][:, None] * expert_ffn(x[rows], ex.wg_hat, ex.wu_hat, ex.wd_hat)
    return out.astype(np.float32)


def plan_tiers(hot, bytes_per_tier, budget_bytes: int, hi_tier: int, lo_tier: int):
    """[DynaExq] (abstract): the experts kept at high precision are chosen by
    usage rank within a memory budget.  Reading: rank experts by hotness (descending,
    ties to the lower id); the n hottest take hi_tier, the rest lo_tier, with n
    the largest count whose total bytes fit the budget.  Returns (tiers, n);
    raises ValueError when all experts at lo_tier already exceed it."""
    E = len(hot)
    lo, hi = int(bytes_per_tier[lo_tier]), int(bytes_per_tier[hi_tier])
    if E * lo > budget_bytes:
        raise ValueError("budget below the all-low-tier size")
    rank = sorted(range(E), key=lambda e: (-float(hot[e]), e))
    n = 0
    while n < E and (n + 1) * hi + (E - n - 1) * lo <= budget_bytes:
        n += 1
    tiers = [lo_tier] * E
    for e in rank[:n]:
        tiers[e] = hi_tier
    return tiers, n


class OracleLayer:
    """A layer's geometry, tier table and lazily built dequantized experts."""

    def __init__(self, hidden: int, inter: int, n_experts: int, top_k: int,
                 tiers: np.ndarray, expert_source):
        """expert_source(e) -> (w_gate, w_up, w_down) bf16 bit arrays."""
        self.H, self.I, self.E, self.k = hidden, inter, n_experts, top_k
        self.tiers = np.asarray(tiers)
        self._src = expert_source
        self._cache: Dict[int, OracleExpert] = {}

    def _build(self, e: int) -> OracleExpert:
        wg, wu, wd = self._src(e)
        return make_expert(int(self.tiers[e]), wg, wu, wd)

    def expert(self, e: int) -> OracleExpert:
        e = int(e)
        if e not in self._cache:
            self._cache[e] = self._build(e)
        return self._cache[e]

    def forward(self, x_bf16, wr_bf16, bias=None, token_subset=None, keep=True):
        """(y float32 [len(subset), H], routing dict).  keep=False builds each
        expert, uses it and drops it, bounding memory for very large experts."""
        r = route(x_bf16, wr_bf16, bias, self.k)
        get = self.expert if keep else self._build
        return layer_forward(x_bf16, r, get, token_subset), r
