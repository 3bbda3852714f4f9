"""GPU MoE layer forward vs the oracle.

Gate (all configs): max |y_f32 - y_oracle| <= tol * RMS(y_oracle); the bf16
output is bytewise the nearest-even rounding of the f32 output; two runs are
bytewise identical.  The tolerance depends on the grouped-GEMM path the
library takes for the call (moe_layer_plan):
  * few routes per expert (path 1): exact integer weight operands and fp32
    sums, so the result differs from the oracle only by summation order and by
    the bf16 rounding of an activation whose fp32 value (a few fp32 ulps from
    the oracle's) lands on the other side of a rounding boundary: one bf16 ulp
    (at most 2^-7 relative) on a few activations.  One such step of the
    largest activation, through a routing weight and a down-projection weight,
    moves an output by about 3e-3 of its RMS at the Qwen3-80B shape (I = 512,
    k = 10, the smallest output RMS per activation); measured up to 2.7e-3
    there, 2.0e-3 or less elsewhere.  Gate: 4e-3;
  * many routes per expert (path 2): the dequantized weight is rounded once to
    fp16 (2^-11 relative per weight), within the 1e-2 layer gate.
Small configs compare every output; the largest compare every token that owns
the first or the last row of an M-tile (so every M-tile and column block of
both GEMMs is checked), at full size, in the launch configuration the
benchmark times.  The log names each case's path and its error.
"""

import dataclasses

import numpy as np
import pytest

import inputs
import oracle
from tests._harness import (Setup, bf16_dev_to_np, log, record_margin, rel_err,
                            tile_boundary_tokens, to_dev)

pytestmark = pytest.mark.gpu

TOL = {1: 4e-3, 2: 1e-2}   # by moe_layer_plan path


def _run(st: Setup, layer=None, subset=None, keep=True, runs=2):
    """subset: None (every token), a list of tokens, or "tiles" (the tokens
    owning the first and the last row of every M-tile)."""
    import torch
    if layer is None:
        layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    (path13, bm13), (path2, bm2) = layer.plan_gemms(st.T)
    path = max(path13, path2)         # the tolerance of the looser GEMM
    log(f"forward cfg{st.cfg.cid} T={st.T} tiers={np.bincount(st.tiers, minlength=3).tolist()} "
        f"gate/up path={path13} tile_rows={bm13}, down path={path2} tile_rows={bm2}")
    y32 = layer.forward(x, wr, b, out_dtype=torch.float32)
    y16 = layer.forward(x, wr, b, out_dtype=torch.bfloat16)
    y32b = layer.forward(x, wr, b, out_dtype=torch.float32) if runs > 1 else y32
    torch.cuda.synchronize()
    y32n, y32bn = y32.cpu().numpy(), y32b.cpu().numpy()
    y16n = bf16_dev_to_np(y16)
    assert np.array_equal(y32n.view(np.uint32), y32bn.view(np.uint32)), "not deterministic"
    assert np.array_equal(y16n, oracle.f32_to_bf16_rne(y32n)), "bf16 output != RNE(f32 output)"
    ol = st.oracle_layer()
    r = oracle.route(st.x, st.wr, st.bias, st.k)
    if isinstance(subset, str):
        subset = np.union1d(tile_boundary_tokens(r, st.E, bm13), tile_boundary_tokens(r, st.E, bm2))
        log(f"  comparing {len(subset)} tokens: the first and last row of every M-tile of both GEMMs")
    get = ol.expert if keep else ol._build
    y_ref = oracle.layer_forward(st.x, r, get, subset)
    got = y32n if subset is None else y32n[subset]
    err = rel_err(got, y_ref)
    got16 = oracle.bf16_bits_to_f32(y16n if subset is None else y16n[subset])
    log(f"  path {path}: max|err|/rms f32 = {err:.3e} (tol {TOL[path]:.1e})   "
        f"bf16 output = {rel_err(got16, y_ref):.3e}")
    record_margin(f"H{st.H} E{st.E} k{st.k} I{st.I} T={st.T} "
                  f"tiers={np.bincount(st.tiers, minlength=3).tolist()} tiles={bm13}/{bm2}"
                  + ("" if subset is None else f" ({len(subset)} tokens)"), path, err, TOL[path])
    assert err <= TOL[path]
    return layer, y32n


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_layer_small_configs_full(cid):
    _run(Setup(cid))


@pytest.mark.parametrize("T", [32, 64, 128, 256, 512])
def test_layer_olmoe_full(T):
    """The OLMoE-shaped layer (H 2048, E 64, top-8, I 1024): decode with 8-row
    tiles (T 32), with 16-row tiles staged in two K-chunks (T 64: 8 rows per
    expert on average), with 64-row tiles (T 128, 256: 16 and 32 rows per
    expert, ragged), and the large-batch path (T 512)."""
    _run(Setup(6, T=T))


@pytest.mark.parametrize("T", [40, 80, 200])
def test_layer_mixed_tiers_skewed_decode(T):
    """Qwen3-30B shape with bf16, int8 and int4 experts and the Zipf bias at
    2.5, 5 and 12.5 rows per expert on average: 8-, 16- and 64-row decode
    tiles, hot experts spanning several tiles (their tiles grouped by XCD)."""
    _run(Setup(3, T=T), keep=False)


@pytest.mark.parametrize("T", [1, 32, 256])
def test_layer_qwen80b_sweep_full(T):
    _run(Setup(4, T=T), keep=False)


@pytest.mark.parametrize("T", [1024, 2048])
def test_layer_qwen80b_mid_full(T):
    """512 experts at 20 and 40 rows per expert on average: the decode kernels
    with 64-row tiles (row blocks past an expert's routes skipped, the rows
    staged into LDS by DMA); every output compared."""
    assert Setup(4, T=8).gpu_layer(experts=[0]).plan_gemms(T) == ((1, 64), (1, 64))
    _run(Setup(4, T=T), keep=False)


@pytest.mark.parametrize("T", [3584, 4096])
def test_layer_qwen80b_mixed_plan_tiles(T):
    """70 and 80 rows per expert: the large-batch gate/up GEMM (row-aware
    partial tiles) writes bf16 activations and their 32-column row sums for
    the decode down GEMM with 64-row tiles (experts spanning two); the first
    and last row of every M-tile of both GEMMs compared."""
    st = Setup(4, T=T)
    layer = st.gpu_layer()
    assert layer.plan_gemms(T) == ((2, 256), (1, 64))
    _run(st, layer=layer, subset="tiles", keep=False)


def test_layer_mixtral_prefill_tiles():
    """8192 tokens on 8 experts: 256-row tiles, the down GEMM's XCD block
    remap (K = I = 14336); the first and last row of every M-tile compared."""
    _run(Setup(5), subset="tiles", keep=False, runs=2)


@pytest.mark.parametrize("T", [1, 32, 64])
def test_layer_mixtral_decode_sampled(T):
    """Mixtral shape at decode sizes: the down GEMM's K = 14336 is staged in
    K-chunks: four with 8-row tiles at T = 1 (the last one partial),
    fourteen with 16-row tiles at T = 32, twenty-eight with 32-row tiles at
    T = 64."""
    _run(Setup(5, T=T), subset="tiles", keep=False, runs=2)


def test_layer_decode_ragged_k_chunks():
    """Both decode GEMMs with K just past one staged chunk (hidden 4352 and
    inter 4224: a last chunk of two k-groups and of one), over all tiers."""
    c = dataclasses.replace(inputs.get_config(1), hidden=4352, inter=4224, n_experts=4,
                            top_k=2, max_tokens=16)
    _run(Setup(1, T=16, cfg=c, tiers=np.array([2, 1, 0, 2])), keep=False)


@pytest.mark.parametrize("T", [65, 100, 128, 129, 200])
def test_layer_large_batch_ragged_k(T):
    """A layer whose K-chunk counts are odd (hidden 4352, inter 4224: 34 and
    33 steps of two 64-wide chunks), all routes on experts 0 (int4) and 3
    (int8) at T rows each.  With four experts the decode launches would have
    few waves, so past 28 mean rows per expert (every T here) the
    large-batch kernels run: int4 tiles of at most 128 rows split K between
    the block's two wave rows (the down GEMM with a last single step), larger
    ones split rows."""
    c = dataclasses.replace(inputs.get_config(1), hidden=4352, inter=4224, n_experts=4,
                            top_k=2, max_tokens=200)
    b = np.zeros(4, np.float32)
    b[[0, 3]] = 100.0
    st = Setup(1, T=T, cfg=c, bias=b, tiers=np.array([2, 0, 2, 1]))
    layer = st.gpu_layer(experts=[0, 3])
    assert layer.plan_gemms(T) == ((2, 256), (2, 256))
    _run(st, layer=layer, keep=False, runs=1)


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_layer_single_tier(tier):
    st = Setup(1, tiers=np.full(8, tier))
    _run(st)


def test_layer_mixed_tiers_small():
    st = Setup(1, tiers=np.array([0, 1, 2, 2, 1, 0, 2, 1]))
    _run(st)


@pytest.mark.parametrize("T", [1, 2, 3, 15, 16, 17, 31, 33, 64, 65, 127, 128,
                               129, 191, 255, 256, 257])
def test_token_group_sizes(T):
    """All T tokens routed to experts 2 and 5 (large bias): one group of T rows
    per expert, T = 1..128 (the token-group sizes the ExactMoE kernel tests
    cover, section 5.3), across the tile boundaries of both GEMMs.  The plan
    sees T / 4 routes per expert on average (8 experts, top-2) and few decode
    waves: 8-row tiles up to T = 16, split-K 16-row tiles up to T = 112, and
    past that the large-batch kernel, whose partial tiles skip the 16-row
    blocks and weight loads past the group (129..257: both halves of the
    256-row tile, a full tile, a full tile plus one row)."""
    cfg = dataclasses.replace(inputs.get_config(1), max_tokens=300)
    b = np.zeros(8, np.float32)
    b[[2, 5]] = 100.0
    st = Setup(1, T=T, cfg=cfg, bias=b, tiers=np.array([2, 2, 2, 1, 2, 0, 2, 2]))
    _run(st, runs=1)


def test_k_equals_e_and_single_expert():
    c = dataclasses.replace(inputs.get_config(1), top_k=8)
    _run(Setup(1, T=24, cfg=c))
    c1 = dataclasses.replace(inputs.get_config(1), n_experts=1, top_k=1)
    _run(Setup(1, T=24, cfg=c1))


def test_max_experts_and_top_k():
    """The library's limits: 1024 experts (one grouping thread each, 16
    expert slots per top-k lane) and top-16 routing, on a small hidden size;
    routing bit-exact and the layer within the gate."""
    import torch
    c = dataclasses.replace(inputs.get_config(1), hidden=256, inter=128, n_experts=1024,
                            top_k=16, max_tokens=40)
    st = Setup(1, T=40, cfg=c)
    layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    got = {k: v.cpu().numpy() for k, v in layer.route(x, wr, b).items()}
    torch.cuda.synchronize()
    ref = oracle.route(st.x, st.wr, st.bias, st.k)
    assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32))
    for key in ("ids", "offsets", "sorted_routes", "route_pos"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.max(np.abs(got["weights"] - ref["weights"])) <= 1e-6
    _run(st, layer=layer, keep=False)


def test_zero_tokens():
    import torch
    st = Setup(1, T=1)
    layer = st.gpu_layer(experts=[0])
    x = torch.empty((0, st.H), dtype=torch.int16, device="cuda:0")
    wr = to_dev(st.wr)
    y = layer.forward(x, wr, None)
    torch.cuda.synchronize()
    assert y.shape == (0, st.H)
    # routing no tokens writes only the expert offsets, all zero (a fill
    # kernel); the block the allocator hands out held sevens just before
    junk = torch.full((st.E + 1,), 7, dtype=torch.int32, device="cuda:0")
    del junk
    r = layer.route(x, wr, None)
    torch.cuda.synchronize()
    assert r["offsets"].cpu().tolist() == [0] * (st.E + 1)


def test_workspace_too_small():
    import torch
    import mixed_precision_moe_amd as mm
    st = Setup(1, T=8)
    layer = st.gpu_layer(experts=[0])
    x, wr, b = st.dev_inputs()
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(mm.MoeError) as ei:
        layer.forward(x, wr, b, workspace=ws)
    assert ei.value.status == 4


def test_handle_swap_promotes_expert():
    """DynaExq-style promotion through the stable handle table: re-pointing an
    expert to a bf16 version changes the next forward to that version."""
    import torch
    from mixed_precision_moe_amd import pack_expert
    st = Setup(1)
    layer, y_before = _run(st, runs=1)
    tiers = st.tiers.copy()
    wg, wu, wd = st.source(3)
    w13, w2 = pack_expert(to_dev(wg), to_dev(wu), to_dev(wd), 0)
    layer.set_experts(3, [(0, w13, w2)])
    tiers[3] = 0
    st2 = Setup(1, tiers=tiers)
    _, y_after = _run(st2, layer=layer, runs=1)
    assert not np.array_equal(y_before, y_after)


def test_plan_query():
    """moe_layer_plan names the path and M-tiling of each GEMM: the decode
    batches stream weights (path 1); the Mixtral prefill, and the Mixtral
    shape already past 28 routes per expert (few experts, so few decode
    waves), run on the large-batch kernels (path 2) with 256-row tiles; the
    many-expert Qwen3-80B shape takes 64-row decode tiles up to 60 routes per
    expert and then pairs the large-batch gate/up GEMM with the decode down
    GEMM (its I = 512 is short); the OLMoE shape (I = 1024) goes from 64-row
    tiles straight to the large-batch kernels."""
    assert Setup(2).gpu_layer(experts=[0]).plan(32) == (1, 8)
    mixtral = Setup(5, T=1).gpu_layer(experts=[0])
    assert mixtral.plan(8192) == (2, 256)
    assert mixtral.plan_gemms(64) == ((1, 32), (1, 32))
    assert mixtral.plan_gemms(112) == ((1, 32), (1, 32))
    assert mixtral.plan_gemms(113) == ((2, 256), (2, 256))
    q80 = Setup(4, T=1).gpu_layer(experts=[0])
    assert q80.plan_gemms(1) == ((1, 8), (1, 8))
    assert q80.plan_gemms(512) == ((1, 16), (1, 16))
    assert q80.plan_gemms(3072) == ((1, 64), (1, 64))
    assert q80.plan_gemms(3073) == ((2, 256), (1, 64))
    assert q80.plan_gemms(4096) == ((2, 256), (1, 64))
    olmoe = Setup(6, T=1).gpu_layer(experts=[0])
    assert olmoe.plan_gemms(480) == ((1, 64), (1, 64))
    assert olmoe.plan_gemms(481) == ((2, 256), (2, 256))


def test_large_batch_32bit_offset_limit():
    """A large-batch forward whose SwiGLU activations [T k, I] (16-bit) would
    reach 4 GiB is refused on the host with MOE_ESHAPE, before the workspace
    check; one token fewer passes that check and meets the (deliberately
    small) workspace instead.  Neither call enqueues any work, so the small
    x and y buffers are never read."""
    import torch
    import mixed_precision_moe_amd as mm
    from mixed_precision_moe_amd import _lib
    st = Setup(1, T=8)
    layer = st.gpu_layer(experts=[0])
    x, wr, b = st.dev_inputs()
    T = (1 << 32) // (2 * st.k * st.I)          # T k I 2 bytes = 4 GiB
    assert layer.plan(T)[0] == 2 and layer.plan(T - 1)[0] == 2
    y = torch.empty((8, st.H), dtype=torch.float32, device=x.device)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=x.device)
    lib = _lib.load()
    s = torch.cuda.current_stream().cuda_stream

    def call(n):
        return lib.moe_layer_forward(layer._h, x.data_ptr(), wr.data_ptr(), None, n, y.data_ptr(),
                                     mm.api.DTYPE_F32, ws.data_ptr(), ws.numel(), s)
    assert call(T) == _lib.MOE_ESHAPE
    assert b"4 GiB" in lib.moe_last_error()
    assert call(T - 1) == _lib.MOE_ENOSPC
    torch.cuda.synchronize()
