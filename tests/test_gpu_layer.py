"""GPU MoE layer forward vs the oracle.

Gate (all configs): max |y_f32 - y_oracle| <= 1e-2 * RMS(y_oracle); the bf16
output is bytewise the nearest-even rounding of the f32 output; two runs are
bytewise identical.  Small configs compare every output; the two largest
compare sampled tokens at their full size in the launch configuration the
benchmark times.
"""

import dataclasses

import numpy as np
import pytest

import inputs
import oracle
from tests._harness import Setup, bf16_dev_to_np, log, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _run(st: Setup, layer=None, subset=None, keep=True, runs=2):
    import torch
    if layer is None:
        layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    log(f"forward cfg{st.cfg.cid} T={st.T} tiers={np.bincount(st.tiers, minlength=3).tolist()}")
    y32 = layer.forward(x, wr, b, out_dtype=torch.float32)
    y16 = layer.forward(x, wr, b, out_dtype=torch.bfloat16)
    y32b = layer.forward(x, wr, b, out_dtype=torch.float32) if runs > 1 else y32
    torch.cuda.synchronize()
    y32n, y32bn = y32.cpu().numpy(), y32b.cpu().numpy()
    y16n = bf16_dev_to_np(y16)
    assert np.array_equal(y32n.view(np.uint32), y32bn.view(np.uint32)), "not deterministic"
    assert np.array_equal(y16n, oracle.f32_to_bf16_rne(y32n)), "bf16 output != RNE(f32 output)"
    ol = st.oracle_layer()
    y_ref, _ = ol.forward(st.x, st.wr, st.bias, token_subset=subset, keep=keep)
    got = y32n if subset is None else y32n[subset]
    err = rel_err(got, y_ref)
    got16 = oracle.bf16_bits_to_f32(y16n if subset is None else y16n[subset])
    log(f"  max|err|/rms f32 = {err:.3e}   bf16 output = {rel_err(got16, y_ref):.3e}")
    assert err <= TOL
    return layer, y32n


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_layer_small_configs_full(cid):
    _run(Setup(cid))


@pytest.mark.parametrize("T", [32, 64, 128, 512])
def test_layer_olmoe_full(T):
    """The OLMoE-shaped layer (H 2048, E 64, top-8, I 1024): decode with 8-row
    tiles (T 32), with 16-row tiles staged in two K-chunks (T 64, 128: 8 and
    16 rows per expert on average), and the large-batch path (T 512)."""
    _run(Setup(6, T=T))


@pytest.mark.parametrize("T", [40, 80, 200])
def test_layer_mixed_tiers_skewed_decode(T):
    """Qwen3-30B shape with bf16, int8 and int4 experts and the Zipf bias at
    2.5, 5 and 12.5 rows per expert on average: 8- and 16-row decode tiles,
    hot experts spanning several tiles (their tiles grouped by XCD)."""
    _run(Setup(3, T=T), keep=False)


@pytest.mark.parametrize("T", [1, 32, 256])
def test_layer_qwen80b_sweep_full(T):
    _run(Setup(4, T=T), keep=False)


def test_layer_qwen80b_1024_sampled():
    """512 experts at 20 rows per expert on average: the decode kernels with
    16-row tiles, experts spanning up to four tiles."""
    st = Setup(4, T=1024)
    sub = [0, 1, 511, 512, 1000, 1023]
    _run(st, subset=sub, keep=False)


def test_layer_qwen80b_4096_sampled():
    st = Setup(4, T=4096)
    sub = list(range(0, 4096, 97))[:40] + [4095]
    _run(st, subset=sub, keep=False)


def test_layer_mixtral_prefill_sampled():
    st = Setup(5)
    sub = [0, 1, 2, 1000, 2047, 2048, 4095, 4096, 6000, 8190, 8191]
    _run(st, subset=sub, keep=False, runs=2)


@pytest.mark.parametrize("T", [1, 32, 64])
def test_layer_mixtral_decode_sampled(T):
    """Mixtral shape at decode sizes: the down GEMM's K = 14336 is staged in
    K-chunks: four with 8-row tiles at T = 1 (the last one partial),
    fourteen with 16-row tiles at T = 32, twenty-eight with 32-row tiles at
    T = 64."""
    st = Setup(5, T=T)
    sub = [0] if T == 1 else [0, T - 1]
    _run(st, subset=sub, keep=False, runs=2)


def test_layer_decode_ragged_k_chunks():
    """Both decode GEMMs with K just past one staged chunk (hidden 4352 and
    inter 4224: a last chunk of two k-groups and of one), over all tiers."""
    c = dataclasses.replace(inputs.get_config(1), hidden=4352, inter=4224, n_experts=4,
                            top_k=2, max_tokens=16)
    _run(Setup(1, T=16, cfg=c, tiers=np.array([2, 1, 0, 2])), keep=False)


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
    cover, section 5.3), across the tile boundaries of both GEMMs; past 32
    routes per expert the large-batch kernel runs, whose partial tiles skip
    the 16-row blocks and weight loads past the group (129..257: both halves
    of the 256-row tile, a full tile, a full tile plus one row)."""
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
