"""Benchmark of the quantized MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

One step is one whole layer forward (routing, grouping, gate/up GEMM + SwiGLU,
down GEMM, combine) over one batch of synthetic tokens already resident in
HBM.  The default workload is the Qwen3-30B-A3B-shaped decode layer
(H 2048, E 128, top-8, I 768, all experts int4 group-128, 32 tokens).  Weight
sets are rotated across R device copies so consecutive steps do not re-read
weights from the 256 MB last-level cache.

Prints one JSON line: whole-job tokens/s, the dominant kernel's roofline
(algorithmic bytes or flops per launch over its measured average duration,
from HIP events recorded on the forward's stream inside the timed region),
and the CPU oracle timed on a bounded sample as a baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import inputs  # noqa: E402

METRIC = "MoE-layer tokens/s; % HBM roofline (decode) and % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s
STAGES = ["route_logits", "topk", "grouping", "gemm_gate_up_swiglu", "gemm_down", "combine"]
CSRC = os.path.join(ROOT, "mixed_precision_moe_amd", "csrc")
# sources of the dominant kernel of each path (a change voids stored counters)
KERNEL_SOURCES = {"decode": ("grouped_gemm.hip", "device_util.h"),
                  "prefill": ("gemm_prefill.hip", "device_util.h")}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def packed_bytes(tier, n, k):
    if tier == 2:
        return n * k // 2 + n * (k // 128) * 2
    if tier == 1:
        return n * k + 2 * n
    return 2 * n * k


def _code_only(text: str) -> str:
    """C/HIP source with comments removed and whitespace collapsed, so that
    a comment edit does not change the hash of the code it describes."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(path_kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path_kind]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def build_layers(cfg, tiers, R, dev):
    """R Layer objects over R distinct device copies of the packed experts."""
    import torch
    import mixed_precision_moe_amd as mm
    blobs = []
    for e in range(cfg.n_experts):
        wg, wu, wd = inputs.gen_expert(cfg, e)
        t = [torch.from_numpy(a.view(np.int16)).to(dev) for a in (wg, wu, wd)]
        blobs.append(mm.pack_expert(*t, int(tiers[e])))
        del t
    layers = []
    for r in range(R):
        hs = []
        for e in range(cfg.n_experts):
            w13, w2 = blobs[e] if r == 0 else (blobs[e][0].clone(), blobs[e][1].clone())
            hs.append((int(tiers[e]), w13, w2))
        layers.append(mm.Layer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, hs))
    torch.cuda.synchronize()
    return layers


def algorithmic(cfg, tiers, ids, T):
    """Algorithmic bytes and flops of the two grouped GEMMs for this routing."""
    touched = np.unique(ids)
    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    w13 = sum(packed_bytes(int(tiers[e]), 2 * I, H) for e in touched)
    w2 = sum(packed_bytes(int(tiers[e]), H, I) for e in touched)
    b13 = w13 + 2 * T * H + 2 * T * k * I            # weights + x in + activation out
    b2 = w2 + 2 * T * k * I + 4 * T * k * H          # weights + activation in + rows out
    f13 = 2.0 * T * k * H * 2 * I
    f2 = 2.0 * T * k * I * H
    router = 2 * cfg.n_experts * H
    return dict(touched=int(touched.size), bytes13=b13, bytes2=b2, flops13=f13, flops2=f2,
                bytes_layer=w13 + w2 + 4 * T * H + router, flops_layer=f13 + f2)


def cpu_baseline(cfg, tiers, x, wr, bias, min_seconds=10.0, max_seconds=30.0):
    """The oracle forward (dequantize touched experts, route, expert FFNs,
    combine) timed on this host over the same synthetic batch."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                                   # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    r0 = oracle.route(x, wr, bias, cfg.top_k)
    touched = np.unique(r0["ids"])
    pre = {}
    for e in touched:                                     # quantization is not timed
        wg, wu, wd = inputs.gen_expert(cfg, int(e))
        w13 = np.concatenate([wg, wu], axis=0)
        t = int(tiers[e])
        pre[int(e)] = (t, oracle.quantize_tier(t, w13), oracle.quantize_tier(t, wd), w13, wd)
    I = cfg.inter

    def get(e):
        t, (q13, s13), (q2, s2), w13, wd = pre[e]
        w13h = oracle.dequantize(t, q13, s13, w13)
        return oracle.OracleExpert(t, w13h[:I], w13h[I:], oracle.dequantize(t, q2, s2, wd))

    import contextlib
    ctx = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        reps, t0 = 0, time.perf_counter()
        while True:
            r = oracle.route(x, wr, bias, cfg.top_k)
            oracle.layer_forward(x, r, get)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or el * (reps + 1) / reps > max_seconds:
                break
    T = x.shape[0]
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(T * reps / el, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model,
            "sample": f"{reps} full forward(s) of the same {T}-token batch (dequantize "
                      f"{touched.size} touched experts, route, expert FFNs, combine; "
                      f"quantization excluded); numpy float64, BLAS pool of {cores} threads",
            "seconds": round(el, 2)}


def stored_traffic(workload_key, path_kind):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter runs (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy of known
    size), if they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path)).get(workload_key)
    except (ValueError, OSError):
        return None
    if not d or d.get("source_sha") != source_hash(path_kind):
        return None
    return d.get("traffic_bytes")


def compare_sequential(layer, x, wr, bias, ids, T, H, dev, fused_fwd, reps):
    """The layer-level comparison the ExactMoE page makes (sequential per-expert
    execution vs one fused grouped forward), on MI355X: the same layer, the
    same tokens, either one fused forward, or one wave per touched expert (the
    slot map sends only that expert to its slot; the first wave routes, the
    others keep its routing and accumulate).  Both are host-launched and timed
    with events; the accumulated output is checked against the fused one."""
    import torch
    touched = sorted(set(int(e) for e in np.unique(ids)))
    E = layer.n_experts
    layer.set_slots(0, layer.handles)            # slot e holds expert e
    maps = []
    for e in touched:
        m = [-1] * E
        m[e] = e
        maps.append(m)
    y_seq = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = layer.workspace(T, dev)

    def sequential():
        for i, m in enumerate(maps):
            layer.set_slot_map(m)
            layer.forward_wave(x, wr, bias, y=y_seq, accumulate=i > 0, workspace=ws)

    y_fused = layer.forward(x, wr, bias, out_dtype=torch.float32)
    sequential()
    torch.cuda.synchronize()
    gap = float((y_seq - y_fused).abs().max() / y_fused.pow(2).mean().sqrt())
    times = {}
    for name, fn in (("fused", fused_fwd), ("sequential", sequential)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        times[name] = a.elapsed_time(b) / reps
    log(f"[bench] fused {times['fused']:.3f} ms, sequential over {len(touched)} experts "
        f"{times['sequential']:.3f} ms; outputs agree to {gap:.1e} x RMS")
    return {"fused_ms_per_layer": round(times["fused"], 4),
            "sequential_ms_per_layer": round(times["sequential"], 4),
            "fused_speedup": round(times["sequential"] / times["fused"], 2),
            "experts_run_one_at_a_time": len(touched),
            "max_abs_gap_over_rms": gap,
            "launch": "host launch per call, both",
            "sequential_kind": "one wave per touched expert: slot-map update, regroup, gate/up GEMM, "
                               "down GEMM, accumulate"}


def dense_gemm_reference(M, K, N, dev, reps=20):
    """Context for an MFMA-bound gate/up kernel: the vendor library's dense
    GEMM (torch.matmul, i.e. hipBLASLt) on the same total shape [M, K] x
    [K, N], in fp16 and bf16, timed with events on this GPU.  It has no
    grouping, gathering, dequantization or epilogue, so it bounds what a
    16-bit MFMA GEMM of this size reaches here at this GPU's sustained clock."""
    import torch
    res = {"library": "torch.matmul (hipBLASLt)", "shape_mkn": [M, K, N]}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for name, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        a = torch.randn(M, K, device=dev, dtype=dt, generator=g)
        b = torch.randn(K, N, device=dev, dtype=dt, generator=g)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            c = a @ b
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / reps * 1000.0
        res[f"{name}_us"] = round(us, 1)
        res[f"{name}_tflops"] = round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1)
        del a, b, c
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=sorted(inputs.CONFIGS))
    ap.add_argument("--tokens", type=int, default=None, help="token count (default: the config's)")
    ap.add_argument("--rotate", type=int, default=None, help="weight-set copies (default: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--eager", action="store_true",
                    help="launch each forward from the host instead of replaying a HIP graph")
    ap.add_argument("--compare-sequential", action="store_true",
                    help="also time the same layer run one expert at a time (per-expert waves "
                         "through the slot map) against the fused grouped forward")
    ap.add_argument("--no-dense-reference", action="store_true",
                    help="skip timing the vendor dense GEMM of the same total shape beside an "
                         "MFMA-bound gate/up kernel")
    ap.add_argument("--prefill-config", type=int, default=5,
                    help="also measure this config at its default token count as the large-batch "
                         "record ('prefill' in the JSON); 0 to skip")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run plain device copies of this many MiB (for scaling HBM "
                         "counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the layer is measured on "
              f"a single MI355X; multi-GPU sharding is described in the design notes, not run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mixed_precision_moe_amd as mm  # noqa: F401
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(10):
            dst.copy_(src)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / 10
        log(f"[bench] copied {n} bytes x 13 (read {n}, write {n} per copy); "
            f"{ms * 1e3:.1f} us per copy = {2 * n / ms / 1e6:.0f} GB/s read+write")
        return
    cfg = inputs.get_config(args.config)
    T = cfg.default_tokens if args.tokens is None else args.tokens
    m = measure(cfg, T, args.steps, args.warmup, args, dev)
    out = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": m["config"],
        "roofline": m["roofline"],
    }
    if args.compare_sequential:
        out["comparison"] = compare_sequential(m["layers"][0], m["x"], m["wr"], m["bias"], m["ids"], T,
                                               cfg.hidden, dev, m["fwd"][0],
                                               max(5, min(args.steps, 50)))
    for L in m["layers"]:
        L.close()
    if args.prefill_config and args.prefill_config != args.config:
        # the large-batch record: the Mixtral-shaped 8192-token prefill, where
        # the gate/up kernel is MFMA-bound; timed the same way, fewer steps
        pcfg = inputs.get_config(args.prefill_config)
        pm = measure(pcfg, pcfg.default_tokens, max(4, min(args.steps, args.prefill_steps)),
                     min(args.warmup, 3), args, dev)
        for L in pm["layers"]:
            L.close()
        out["prefill"] = {"value": pm["value"], "unit": "tokens/s", "ms_per_step": pm["ms_per_step"],
                          "steps": pm["steps"], "config": pm["config"], "roofline": pm["roofline"]}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(cfg, m["tiers"], m["x_np"], m["wr_np"], m["bias_np"])
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def measure(cfg, T, steps, warmup, args, dev):
    """Time whole-layer forwards of one workload: a host-launched region with
    per-stage events (and the gate/up kernel's own start and end), then a HIP
    graph of R forwards (one per weight copy) replayed back to back, from which
    the throughput is taken."""
    import torch
    tiers = inputs.gen_tiers(cfg)
    x_np, wr_np, bias_np = inputs.gen_tokens(cfg, T), inputs.gen_router(cfg), inputs.gen_bias(cfg)
    total_w = sum(packed_bytes(int(tiers[e]), 2 * cfg.inter, cfg.hidden) +
                  packed_bytes(int(tiers[e]), cfg.hidden, cfg.inter) for e in range(cfg.n_experts))
    R = args.rotate or max(1, min(16, int(np.ceil(1.0e9 / total_w))))
    log(f"[bench] {cfg.describe(T)}; weights {total_w / 1e6:.1f} MB x {R} rotating copies")
    t0 = time.time()
    layers = build_layers(cfg, tiers, R, dev)
    log(f"[bench] packed in {time.time() - t0:.1f} s")

    x = torch.from_numpy(x_np.view(np.int16)).to(dev)
    wr = torch.from_numpy(wr_np.view(np.int16)).to(dev)
    bias = None if bias_np is None else torch.from_numpy(bias_np).to(dev)
    ydt = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    y = torch.empty((T, cfg.hidden), dtype=ydt, device=dev)
    ws = torch.empty(layers[0].workspace_size(T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    fwd = [L.bind_forward(x, wr, bias, y, workspace=ws, stream=stream) for L in layers]
    (path, tile_rows), (path2, tile_rows2) = layers[0].plan_gemms(T)

    # routing (for the algorithmic byte/flop counts): outside the timed region
    route = layers[0].route(x, wr, bias)
    ids = route["ids"].cpu().numpy()
    del route
    alg = algorithmic(cfg, tiers, ids, T)

    for i in range(warmup):
        fwd[i % R]()
    torch.cuda.synchronize()

    K = steps
    # Timed region 1: one host launch per forward, HIP events recorded on the
    # forward's stream around every stage (the per-kernel durations).
    # events 0..6: stage boundaries; 7, 8: the gate/up GEMM kernel's own start
    # and end (timestamps of that kernel's dispatch, without stage gaps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(9)] for _ in range(K)]
    for i in range(K):                     # create the events before the timed region
        for e in ev[i]:
            e.record(stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        layers[i % R].set_stage_events(ev[i])
        fwd[i % R]()
    end.record(stream)
    torch.cuda.synchronize()
    for L in layers:
        L.set_stage_events(None)
    eager_ms = start.elapsed_time(end)
    stage_ms = np.array([[ev[i][s].elapsed_time(ev[i][s + 1]) for s in range(6)] for i in range(K)])
    g13_kernel_us = float(np.mean([ev[i][7].elapsed_time(ev[i][8]) for i in range(K)]) * 1000)
    total_ms, launch = eager_ms, "host launch per forward"
    warm_ms = None
    if not args.eager:
        # Timed region 2: one HIP graph holds R forwards (one per weight copy);
        # the region replays it back to back.  Throughput is taken from here.
        K = max(R, (K // R) * R)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for r in range(R):
                layers[r].bind_forward(x, wr, bias, y, workspace=ws, stream=cap)()
        graph.replay()                     # one untimed replay
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(K // R):
            graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        total_ms, launch = start.elapsed_time(end), f"HIP graph of {R} forwards, replayed"
        del graph
        # Labelled context, never the value: the same weight set every step
        # (its weights stay in the 256 MB last-level cache where they fit).
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for r in range(R):
                layers[0].bind_forward(x, wr, bias, y, workspace=ws, stream=cap)()
        graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(K // R):
            graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        warm_ms = start.elapsed_time(end) / K
        del graph
    stage_avg_us = (stage_ms.mean(axis=0) * 1000).round(2)
    ms_per_step = total_ms / K
    value = T * K / (total_ms / 1000.0)
    log(f"[bench] {ms_per_step * 1000:.2f} us per layer; gate/up GEMM kernel (own timestamps): "
        f"{g13_kernel_us:.2f} us")
    log("[bench] stage averages (us): " +
        ", ".join(f"{n}={v}" for n, v in zip(STAGES, stage_avg_us)))

    # the kernel is MFMA-bound when its flops take longer at peak than its bytes
    prefill = alg["flops13"] / (BF16_PEAK_TFLOPS * 1e12) > alg["bytes13"] / (HBM_PEAK_GBS * 1e9)
    g13_s = g13_kernel_us * 1e-6
    workload_key = f"cfg{cfg.cid}_T{T}"
    if prefill:
        achieved = alg["flops13"] / g13_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = alg["bytes13"] / g13_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = "grouped_gemm gate/up + SwiGLU"
    roof["avg_launch_us"] = round(g13_kernel_us, 3)
    roof["timing"] = ("HIP events carried by the kernel's own dispatch (hipExtLaunchKernelGGL) on the "
                      "forward's stream, averaged over the host-launched timed region")
    roof["algorithmic_per_launch"] = alg["flops13"] if prefill else alg["bytes13"]
    roof["traffic"] = stored_traffic(workload_key, "prefill" if prefill else "decode")
    if prefill and not args.no_dense_reference:
        ref = dense_gemm_reference(T * cfg.top_k, cfg.hidden, 2 * cfg.inter, dev)
        ref["kernel_vs_f16"] = round(achieved / ref["f16_tflops"], 3)
        roof["dense_gemm_reference"] = ref
        log(f"[bench] dense f16 GEMM of the same total shape: {ref['f16_tflops']} TFLOP/s "
            f"(bf16 {ref['bf16_tflops']}); the gate/up kernel reaches {ref['kernel_vs_f16']} of it")

    layer_roof_s = max(alg["bytes_layer"] / (HBM_PEAK_GBS * 1e9),
                       alg["flops_layer"] / (BF16_PEAK_TFLOPS * 1e12))
    config = {
        "workload": cfg.describe(T),
        "tokens": T, "hidden": cfg.hidden, "experts": cfg.n_experts, "top_k": cfg.top_k,
        "inter": cfg.inter, "touched_experts": alg["touched"],
        "gemm_path": {1: "few routes per expert (weight streaming)",
                      2: "many routes per expert (fp16 MFMA)"}.get(path, str(path)),
        "tile_rows": tile_rows,
        "down_gemm_path": {1: "few routes per expert (weight streaming)",
                           2: "many routes per expert (fp16 MFMA)"}.get(path2, str(path2)),
        "down_tile_rows": tile_rows2,
        "weight_copies_rotated": R, "output": args.out_dtype,
        "ms_per_step_one_weight_set": None if warm_ms is None else round(warm_ms, 5),
        "one_weight_set_note": ("context only: the same weight copy every step, so weights may be "
                                "served by the last-level cache; value rotates the copies"),
        "launch": launch, "ms_per_step_host_launch": round(eager_ms / steps, 4),
        "layer_roofline_frac": round(layer_roof_s / (ms_per_step / 1000.0), 4),
        "layer_bound": "mfma" if alg["flops_layer"] / (BF16_PEAK_TFLOPS * 1e12) >
                       alg["bytes_layer"] / (HBM_PEAK_GBS * 1e9) else "hbm",
        "stage_avg_us": dict(zip(STAGES, [float(v) for v in stage_avg_us])),
    }
    return dict(value=round(value, 1), steps=K, ms_per_step=round(ms_per_step, 5), config=config,
                roofline=roof, layers=layers, fwd=fwd, x=x, wr=wr, bias=bias, ids=ids, tiers=tiers,
                x_np=x_np, wr_np=wr_np, bias_np=bias_np)


if __name__ == "__main__":
    main()
