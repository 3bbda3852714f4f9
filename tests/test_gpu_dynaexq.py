"""DynaExq online loop on the GPU ("Dynamic Expert Quantization for Scalable
Mixture-of-Experts Inference", abstract): usage counted from the routing,
budgeted plan of the most used experts, asynchronous repack, promotion through the stable
handle table.

* The hotness trace equals the oracle's route counts exactly (plain counts and
  a power-of-two decay are exact in fp32).
* The stream-ordered repack writes the same bytes as the synchronous one.
* After a replan the promoted set is the oracle plan's, forwards enqueued
  before the swap run on the old versions and forwards after it match the
  oracle layer with the new tiers.
"""

import numpy as np
import pytest

import inputs
import oracle
from tests._harness import Setup, log, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _counts(st):
    r = oracle.route(st.x, st.wr, st.bias, st.k)
    return np.bincount(r["ids"].ravel(), minlength=st.E).astype(np.float32)


def test_hotness_trace_counts_routes():
    import torch
    st = Setup(1, T=64)
    layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    c = _counts(st)
    hot = torch.zeros(st.E, dtype=torch.float32, device=x.device)
    layer.set_hotness(hot, 1.0)
    for _ in range(3):
        layer.forward(x, wr, b)
    layer.route(x, wr, b)                      # routing alone does not count
    torch.cuda.synchronize()
    assert np.array_equal(hot.cpu().numpy(), 3 * c)
    hot.zero_()
    layer.set_hotness(hot, 0.5)
    layer.forward(x, wr, b)
    layer.forward(x, wr, b)
    torch.cuda.synchronize()
    assert np.array_equal(hot.cpu().numpy(), 1.5 * c)
    # waves: only the first wave of a layer call (accumulate = 0) counts
    hot.zero_()
    layer.set_hotness(hot, 1.0)
    y = torch.zeros((st.T, st.H), dtype=torch.float32, device=x.device)
    layer.forward_wave(x, wr, b, y=y)
    layer.forward_wave(x, wr, b, y=y, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(hot.cpu().numpy(), c)
    layer.set_hotness(None)
    layer.forward(x, wr, b)
    torch.cuda.synchronize()
    assert np.array_equal(hot.cpu().numpy(), c)


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_async_pack_matches_sync(tier):
    import torch
    from mixed_precision_moe_amd import (LAYOUT_GATE_UP, packed_size, quantize_pack,
                                         quantize_pack_async)
    cfg = inputs.get_config(2)
    wg, wu, _ = inputs.gen_expert(cfg, 5)
    w = to_dev(np.concatenate([wg, wu], axis=0))
    ref = quantize_pack(w, tier, LAYOUT_GATE_UP)
    out = torch.full((packed_size(tier, *w.shape),), 0xAB, dtype=torch.uint8, device=w.device)
    status = torch.full((1,), 7, dtype=torch.int32, device=w.device)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        quantize_pack_async(w, tier, LAYOUT_GATE_UP, out, status, s)
    s.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, ref)
    if tier != 0:
        bad = w.clone()
        bad[3, 9] = 0x7FC0                     # NaN
        quantize_pack_async(bad, tier, LAYOUT_GATE_UP, out, status)
        torch.cuda.synchronize()
        assert int(status.item()) != 0


def test_controller_promotes_the_hot_set():
    import torch
    from mixed_precision_moe_amd import DynaExq, Layer, pack_expert
    c0 = inputs.get_config(1)
    bias = np.zeros(c0.n_experts, np.float32)
    bias[[2, 5, 6]] = [0.6, 0.9, 0.3]          # a skewed router: experts 5, 2, 6 hot
    st = Setup(1, T=64, tiers=np.full(8, 2), bias=bias)
    blobs = []
    for e in range(st.E):
        wg, wu, wd = st.source(e)
        blobs.append((2, *pack_expert(to_dev(wg), to_dev(wu), to_dev(wd), 2)))
    layer = Layer(st.H, st.I, st.E, st.k, blobs)
    x, wr, b = st.dev_inputs()
    masters = {e: tuple(to_dev(a) for a in st.source(e)) for e in range(st.E)}
    ctl = DynaExq(layer, lambda e: masters[e], blobs, budget_bytes=0)
    sizes = ctl.bytes_per_tier()
    ctl.budget = 2 * sizes[0] + (st.E - 2) * sizes[2]     # room for two bf16 experts
    for _ in range(4):
        layer.forward(x, wr, b)
    c = _counts(st)
    want_tiers, n = oracle.plan_tiers((4 * c).tolist(), sizes, ctl.budget, 0, 2)
    log(f"route counts {c.tolist()} -> plan {want_tiers}")
    assert n == 2
    changed = ctl.replan()
    assert sorted(changed) == sorted(e for e in range(st.E) if want_tiers[e] == 0)
    y_old = layer.forward(x, wr, b, out_dtype=torch.float32)   # enqueued before the swap
    ctl.apply(wait=True)
    y_new = layer.forward(x, wr, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert ctl.tiers() == want_tiers
    ref_old, _ = Setup(1, T=64, tiers=np.full(8, 2), bias=bias).oracle_layer().forward(st.x, st.wr, bias)
    st_new = Setup(1, T=64, tiers=np.array(want_tiers), bias=bias)
    ref_new, _ = st_new.oracle_layer().forward(st.x, st.wr, bias)
    e_old, e_new = rel_err(y_old.cpu().numpy(), ref_old), rel_err(y_new.cpu().numpy(), ref_new)
    log(f"  before swap vs int4 oracle {e_old:.2e}; after swap vs planned tiers {e_new:.2e}")
    assert e_old <= 1e-2 and e_new <= 1e-2
    assert rel_err(y_new.cpu().numpy(), ref_old) > e_new     # the promotion changed the result
