"""Wave execution ("Every Expert Counts: ExactMoE ...", §3.4): experts resident
in C < E slots, an explicit global-expert-to-slot map with an inactive
sentinel, one grouped forward per wave, outputs accumulated.

Each wave is compared with the oracle's wave_forward (the same layer with only
the wave's experts contributing); the accumulated waves of a partition of the
experts are compared with the oracle's full layer output and with the
library's single-pass forward.  Gates as for the layer: max |err| <= 1e-2 *
RMS of the full output.
"""

import numpy as np
import pytest

import oracle
from tests._harness import Setup, log, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _packed(st, experts):
    from mixed_precision_moe_amd import pack_expert
    out = {}
    for e in experts:
        wg, wu, wd = st.source(e)
        out[e] = (int(st.tiers[e]), *pack_expert(to_dev(wg), to_dev(wu), to_dev(wd), int(st.tiers[e])))
    return out


def _run_waves(st, n_slots, seed=0):
    import torch
    layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    rng = np.random.default_rng(seed)
    order = rng.permutation(st.E)
    waves = [order[i:i + n_slots] for i in range(0, st.E, n_slots)]
    blobs = _packed(st, range(st.E))
    ol = st.oracle_layer()
    y_full, r = ol.forward(st.x, st.wr, st.bias)
    rms = float(np.sqrt(np.mean(y_full.astype(np.float64) ** 2)))
    y = torch.zeros((st.T, st.H), dtype=torch.float32, device=x.device)
    for wi, wave in enumerate(waves):
        log(f"wave {wi}: {len(wave)} experts in {n_slots} slots (cfg{st.cfg.cid} T={st.T})")
        layer.set_slots(0, [blobs[int(e)] for e in wave])
        smap = [-1] * st.E
        for s_i, e in enumerate(wave):
            smap[int(e)] = s_i
        layer.set_slot_map(smap)
        yw = layer.forward_wave(x, wr, b, out_dtype=torch.float32)
        layer.forward_wave(x, wr, b, y=y, accumulate=True)
        torch.cuda.synchronize()
        ref_w = oracle.wave_forward(st.x, r, ol.expert, wave)
        err_w = float(np.max(np.abs(yw.cpu().numpy().astype(np.float64) - ref_w))) / rms
        log(f"  wave max|err|/rms(full) = {err_w:.3e}")
        assert err_w <= TOL
    yn = y.cpu().numpy()
    err = rel_err(yn, y_full)
    y_one = layer.forward(x, wr, b, out_dtype=torch.float32).cpu().numpy()
    gap = float(np.max(np.abs(yn.astype(np.float64) - y_one))) / rms
    log(f"  accumulated max|err|/rms = {err:.3e}; vs single-pass forward {gap:.3e}")
    assert err <= TOL
    assert gap <= 1e-5          # the same products, summed in a different fp32 order
    return layer


def test_waves_small_layer():
    _run_waves(Setup(1), n_slots=3)


def test_waves_decode_layer():
    _run_waves(Setup(2, T=32), n_slots=48)


def test_waves_prefill_mixed_tiers():
    # 512 tokens of the mixed-tier layer: the large-batch kernels, bf16/int8/int4 slots
    _run_waves(Setup(3, T=512), n_slots=80, seed=3)


def test_sentinel_and_validation():
    import torch
    from mixed_precision_moe_amd import MoeError
    st = Setup(1, T=16)
    layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    # a new layer maps every expert to the sentinel: the wave contributes nothing
    y = layer.forward_wave(x, wr, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not y.cpu().numpy().any()
    y0 = torch.randn((st.T, st.H), device=x.device)
    keep = y0.clone()
    layer.forward_wave(x, wr, b, y=y0, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, keep)
    with pytest.raises(MoeError) as ei:           # slot 0 holds no handle yet
        layer.set_slot_map([0] + [-1] * (st.E - 1))
    assert ei.value.status == 1
    blobs = _packed(st, [2])
    layer.set_slots(0, [blobs[2]])
    with pytest.raises(MoeError) as ei:
        layer.set_slot_map([st.E] + [-1] * (st.E - 1))
    assert ei.value.status == 1
    layer.set_slot_map([-1, -1, 0] + [-1] * (st.E - 3))
    with pytest.raises(MoeError) as ei:           # accumulating into bf16 is refused
        layer.forward_wave(x, wr, b, y=torch.zeros((st.T, st.H), dtype=torch.bfloat16,
                                                   device=x.device), accumulate=True)
    assert ei.value.status == 1


def test_sequential_per_expert_waves_olmoe():
    """The OLMoE-shaped layer run one expert at a time (one wave per touched
    expert, the routing kept from the first) equals the fused forward."""
    import torch
    st = Setup(6, T=32)
    layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    ol = st.oracle_layer()
    y_ref, r = ol.forward(st.x, st.wr, st.bias)
    layer.set_slots(0, layer.handles)
    y = torch.zeros((st.T, st.H), dtype=torch.float32, device=x.device)
    touched = sorted(set(int(e) for e in r["ids"].ravel()))
    for i, e in enumerate(touched):
        m = [-1] * st.E
        m[e] = e
        layer.set_slot_map(m)
        layer.forward_wave(x, wr, b, y=y, accumulate=i > 0)
    y_fused = layer.forward(x, wr, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rms = float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2)))
    gap = float(np.max(np.abs(y.cpu().numpy().astype(np.float64) - y_fused.cpu().numpy()))) / rms
    err = rel_err(y.cpu().numpy(), y_ref)
    log(f"olmoe sequential {len(touched)} waves: vs oracle {err:.2e}, vs fused {gap:.2e}")
    assert err <= TOL and gap <= 1e-5


def test_wave_routing_survives_other_calls_between_waves():
    """A forward() and a route() of other tokens (same T) between a layer
    call's waves do not disturb the routing its accumulating waves reuse, and
    an accumulating wave with no first wave before it is refused."""
    import torch
    st = Setup(2, T=32)
    layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    x_other = to_dev(np.ascontiguousarray(st.x[::-1]))
    layer.set_slots(0, layer.handles)
    half = st.E // 2
    y = torch.zeros((st.T, st.H), dtype=torch.float32, device=x.device)
    layer.set_slot_map([e if e < half else -1 for e in range(st.E)])
    layer.forward_wave(x, wr, b, y=y)
    layer.forward(x_other, wr, b, out_dtype=torch.float32)
    layer.route(x_other, wr, b)
    layer.set_slot_map([e if e >= half else -1 for e in range(st.E)])
    layer.forward_wave(x, wr, b, y=y, accumulate=True)
    torch.cuda.synchronize()
    y_ref, _ = st.oracle_layer().forward(st.x, st.wr, st.bias)
    err = rel_err(y.cpu().numpy(), y_ref)
    log(f"two waves around other calls: max|err|/rms = {err:.3e}")
    assert err <= 2.5e-3
    layer.set_router_mode(0)                     # drops the waves' routing state
    with pytest.raises(ValueError):
        layer.forward_wave(x, wr, b, y=y, accumulate=True)


def test_waves_mixed_plan():
    """Waves on a forward whose plan pairs the large-batch gate/up GEMM with
    the decode down GEMM (128 experts, I 512, 64 routes per expert): one wave
    mapping every expert to itself equals the plain forward bit for bit (the
    same tiles through the slot map), and two half-waves accumulate to it
    within fp32 reordering."""
    import dataclasses
    import torch
    import inputs
    cfg = dataclasses.replace(inputs.get_config(2), inter=512, tokens=(1024,), max_tokens=1024)
    st = Setup(2, T=1024, cfg=cfg)
    layer = st.gpu_layer()
    assert layer.plan_gemms(st.T) == ((2, 256), (1, 64))
    x, wr, b = st.dev_inputs()
    y = layer.forward(x, wr, b, out_dtype=torch.float32)
    layer.set_slots(0, layer.handles)
    layer.set_slot_map(list(range(st.E)))
    y_one = layer.forward_wave(x, wr, b, out_dtype=torch.float32)
    half = st.E // 2
    y_acc = torch.zeros_like(y)
    layer.set_slot_map([e if e < half else -1 for e in range(st.E)])
    layer.forward_wave(x, wr, b, y=y_acc)
    layer.set_slot_map([e if e >= half else -1 for e in range(st.E)])
    layer.forward_wave(x, wr, b, y=y_acc, accumulate=True)
    torch.cuda.synchronize()
    rms = float(torch.sqrt(torch.mean(y.double() ** 2)))
    gap = float(torch.max(torch.abs(y_acc.double() - y.double()))) / rms
    log(f"mixed-plan waves: one wave bitwise {torch.equal(y_one, y)}; two waves vs forward {gap:.2e}")
    assert torch.equal(y_one.view(torch.int32), y.view(torch.int32))
    assert gap <= 1e-5
