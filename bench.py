"""Benchmark of the routed int4 MoE layer on one MI355X.

Default workload: single-token decode through one Gemma-4-26B-A4B-shaped MoE
layer (d_model 2816, 128 experts of GLU width 704 at 4-bit group 64, top-8,
shared expert of width 2112, 8-bit router), bf16 activations.  A step is one
token through one layer: router GEMV + top-8 + gates, fused-dequant GLU of the
8 routed experts and the shared expert, down projection and combine.  Sixteen
seeded replicas of the layer are rotated (6.9 GB of experts resident in HBM,
595 MB touched per rotation) so the 256 MB Infinity Cache cannot hold the
weights; each step takes a fresh seeded token.  Steps are replayed from a HIP
graph.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config decode|prefill|stack30]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synthetic import gen  # noqa: E402

METRIC = "routed-MoE layer tokens/s + achieved HBM GB/s (int4 top-8/128, 1 GPU)"
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_layers(cfg, n_layers, seed, moe, torch):
    layers = []
    nb = gen.blob_bytes(cfg.D, cfg.F)
    for l in range(n_layers):
        host = np.empty((cfg.E, nb), dtype=np.uint8)
        lw = gen.layer_weights(seed, l, cfg, experts_out=host)
        router = moe.DeviceQMat(lw.router.codes, lw.router.meta, cfg.E, cfg.D, 8)
        routed = moe.DeviceBank(torch.from_numpy(host).cuda(), cfg.D, cfg.F)
        shared = moe.DeviceBank.from_numpy(lw.shared[None, :], cfg.D, cfg.F_shared)
        bias = (torch.from_numpy(gen.zipf_bias(seed, l, cfg.E, cfg.beta)).cuda()
                if cfg.beta else None)
        layers.append((router, routed, shared, bias))
    return layers


def cpu_baseline(cfg, seed, budget_s):
    """The oracle as it stands, on the host cores, for a bounded sample."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    lw = gen.layer_weights(seed, 0, cfg)
    bias = gen.zipf_bias(seed, 0, cfg.E, cfg.beta) if cfg.beta else None
    n, t0 = 0, time.perf_counter()
    while True:
        xb = gen.activations(seed, 0, 10_000 + n, cfg.T, cfg.D, cfg.x_dtype)
        O.layer_forward(O.activations_to_float(xb, cfg.x_dtype), lw, cfg.k, bias)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": n * cfg.T / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} calls of {cfg.T} token(s) through layer 0 of the '{cfg.name}' "
                      f"workload in {el:.1f} s (float64 numpy oracle, BLAS threads {threads}, "
                      f"host cpu_count {os.cpu_count()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--config", default="decode", choices=["decode", "prefill", "stack30"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph-steps", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune", action="append", default=[],
                    help="launch-shape knob key=value (moe_set_tuning), repeatable")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_mixture_experts_moe_amd import moe

    torch.cuda.set_device(0)
    for kv in a.tune:
        key, val = kv.split("=")
        moe.moe_set_tuning(key, int(val))
    cfg = gen.CONFIGS[a.config]
    n_layers = cfg.layers
    T = cfg.T
    log(f"config {cfg.name}: generating {n_layers} layer(s)")
    t0 = time.perf_counter()
    layers = build_layers(cfg, n_layers, a.seed, moe, torch)
    log(f"layers resident in HBM ({time.perf_counter() - t0:.1f} s)")
    G = a.graph_steps
    n_x = G
    xb = np.concatenate([gen.activations(a.seed, 1000 + i, 0, T, cfg.D, cfg.x_dtype)
                         for i in range(n_x)])
    x_all = torch.from_numpy(xb.astype(np.int16)).cuda().view(torch.bfloat16).reshape(n_x, T, cfg.D)
    out = torch.empty(n_x, T, cfg.D, dtype=torch.float32, device="cuda")
    ws = moe.Workspace(T, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared)

    def step(i):
        router, routed, shared, bias = layers[i % n_layers]
        moe.moe_layer_forward(x_all[i % n_x], router, cfg.k, routed, shared, out[i % n_x], ws,
                              logit_bias=bias)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(G):  # eager pass (also loads the kernels)
            step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(G):
            step(i)
    torch.cuda.synchronize()
    reps_w = max(1, a.warmup // G)
    reps = max(1, a.steps // G)
    steps = reps * G
    with torch.cuda.stream(stream):
        for _ in range(reps_w):
            graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(reps):
            graph.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / steps
    tokens_per_s = steps * T / (ms / 1e3)
    step_bytes = gen.algorithmic_decode_bytes(cfg) * T if T == 1 else None
    gbps = step_bytes / (ms_step / 1e3) / 1e9 if step_bytes else None
    log(f"{steps} steps in {ms:.2f} ms: {ms_step * 1e3:.2f} us/step, {tokens_per_s:,.0f} tokens/s"
        + (f", {gbps:,.0f} GB/s" if gbps else ""))

    cpu = None
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(cfg, a.seed, a.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": reps_w * G,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations, int4/int8 weights, fp32 accumulate",
        "data": "synthetic (seeded weights and activations)",
        "config": {"workload": f"{cfg.name}: one Gemma-4-26B-A4B-shaped MoE layer, "
                               f"{T} token(s) per step, d_model {cfg.D}, {cfg.E} experts of "
                               f"GLU width {cfg.F} (4-bit, group 64), top-{cfg.k}, shared expert "
                               f"{cfg.F_shared}, 8-bit router; {n_layers} seeded layer replicas "
                               f"rotated", "tokens_per_step": T, "layers_rotated": n_layers,
                   "parallelism": "single GPU"},
        "hbm_GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS if gbps else None, "traffic": None,
                     "kernel": "whole layer step (route, glu, down_combine)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
