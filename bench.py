"""Benchmark of the routed int4 MoE layer on one MI355X.

Default workload: single-token decode through one Gemma-4-26B-A4B-shaped MoE
layer (d_model 2816, 128 experts of GLU width 704 at 4-bit group 64, top-8,
shared expert of width 2112, 8-bit router), bf16 activations.  A step is one
token through one layer: router GEMV + top-8 + gates, fused-dequant GLU of the
8 routed experts and the shared expert, down projection and combine.  Sixteen
seeded replicas of the layer are rotated (6.9 GB of experts resident in HBM,
595 MB touched per rotation) so the 256 MB Infinity Cache cannot hold the
weights; each step takes a fresh seeded token.  Steps are replayed from HIP
graphs of --graph-steps steps (plus one graph of the remainder, so exactly W
warmup and K timed steps run); the median of --regions timed regions of K
steps each is reported.  --block times the residual block around the layer.
Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config decode|prefill|stack30|streamed|store]
                    [--block]
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


def cpu_baseline(cfg, seed, budget_s, block=False):
    """The oracle as it stands, on the host cores, for a bounded sample: the
    workload's own calls with every BLAS thread, one call on one thread, and
    (decode) one 128-token chunk of the prefill workload.  block: the
    oracle's residual block around the layer instead of the layer."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    lw = gen.layer_weights(seed, 0, cfg)
    bias = gen.zipf_bias(seed, 0, cfg.E, cfg.beta) if cfg.beta else None

    w_pre, w_post = gen.norm_weights(seed, 0, cfg.D)

    def calls(budget, stream0):
        n, t0 = 0, time.perf_counter()
        while True:
            if block:
                xb = gen.residual_stream(seed, 0, stream0 + n, cfg.T, cfg.D, cfg.x_dtype)
                O.block_forward(O.activations_to_float(xb, cfg.x_dtype), lw, cfg.k, w_pre,
                                w_post, logit_bias=bias, x_dtype=cfg.x_dtype)
            else:
                xb = gen.activations(seed, 0, stream0 + n, cfg.T, cfg.D, cfg.x_dtype)
                O.layer_forward(O.activations_to_float(xb, cfg.x_dtype), lw, cfg.k, bias)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return n, el

    n, el = calls(budget_s * 0.4, 10_000)
    res = {"value": n * cfg.T / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{n} calls of {cfg.T} token(s) through "
                     + ("the residual block around " if block else "")
                     + f"layer 0 of the '{cfg.name}' "
                     f"workload in {el:.1f} s (float64 numpy oracle, BLAS threads {threads}, "
                     f"host cpu_count {os.cpu_count()})"}
    if threadpool_limits is not None:
        with threadpool_limits(1):
            n1, el1 = calls(budget_s * 0.2, 20_000)
        res["single_thread"] = {"value": n1 * cfg.T / el1, "unit": "tokens/s", "cores": 1,
                                "sample": f"{n1} calls in {el1:.1f} s"}
    if cfg.name == "decode" and not block:
        pc = gen.CONFIGS["prefill"]
        xb = gen.activations(seed, 0, 0, pc.T, pc.D, pc.x_dtype)
        t0 = time.perf_counter()
        O.layer_forward(O.activations_to_float(xb, pc.x_dtype), lw, pc.k,
                        gen.zipf_bias(seed, 0, pc.E, pc.beta))
        elp = time.perf_counter() - t0
        res["prefill_chunk"] = {"value": pc.T / elp, "unit": "tokens/s", "cores": int(threads),
                                "sample": f"one {pc.T}-token chunk (Zipf beta {pc.beta}) in "
                                          f"{elp:.1f} s"}
        res["stack30"] = {"value": res["value"] / 30, "unit": "tokens/s", "cores": int(threads),
                          "sample": "derived: the decode rate over 30 layers of the same shape"}
    return res


# sources that build (and launch) the decode layer kernel: its counters are
# stale once any of them changes
DECODE_LAYER_SOURCES = ("device_common.h", "layer_decode.hip", "moe_api.cpp", "moe_internal.h")


def source_hash(files=DECODE_LAYER_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_mixture_experts_moe_amd", "csrc")
    for f in sorted(files):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(name):
    """HBM bytes per launch of the timed kernel from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), only if they were taken
    on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", name)
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def run_stack(cfg, a, moe, torch):
    """30-layer decode: every token goes through all layers in order."""
    n_layers, n_tok = cfg.layers, cfg.tokens
    log(f"stack: generating {n_layers} layers ({n_layers * cfg.E * gen.blob_bytes(cfg.D, cfg.F) / 1e9:.1f} GB of experts)")
    t0 = time.perf_counter()
    layers = build_layers(cfg, n_layers, a.seed, moe, torch)
    log(f"layers resident in HBM ({time.perf_counter() - t0:.1f} s)")
    xb = np.stack([gen.activations(a.seed, 2000 + l, 0, n_tok, cfg.D, cfg.x_dtype)
                   for l in range(n_layers)])  # [layer, token, D]
    x_all = torch.from_numpy(xb.astype(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty(n_layers, 1, cfg.D, dtype=torch.float32, device="cuda")
    ws = moe.Workspace(1, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared)

    def token(t):
        for l in range(n_layers):
            router, routed, shared, bias = layers[l]
            moe.moe_layer_forward(x_all[l, t:t + 1], router, cfg.k, routed, shared, out[l], ws,
                                  logit_bias=bias)

    G = 8
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for t in range(G):
            token(t)
    torch.cuda.synchronize()
    for g0 in range(0, n_tok, G):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for t in range(g0, g0 + G):
                token(t)
        graphs.append(gr)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graphs[0].replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for gr in graphs:
            gr.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    per_token = gen.algorithmic_decode_bytes(cfg) * n_layers
    res = {"tokens": n_tok, "layers": n_layers, "ms": ms, "tokens_per_s": n_tok / (ms / 1e3),
           "us_per_token": ms * 1e3 / n_tok, "us_per_layer_token": ms * 1e3 / n_tok / n_layers,
           "GBps": per_token * n_tok / (ms / 1e3) / 1e9, "beta": cfg.beta}
    log(f"stack: {res}")
    return res


def run_streamed(cfg, a, moe, torch):
    """30 layers, 16 HBM slots per layer, experts streamed from pinned host
    memory.  --tokens T > 1: each call carries T tokens (a prefill chunk per
    layer, run in slot-sized batches of its experts); --stream-tokens steps."""
    n_layers, n_tok = cfg.layers, a.stream_tokens
    T = a.tokens if a.tokens > 0 else 1
    n_warm = 16 if T == 1 else 2
    nb = gen.blob_bytes(cfg.D, cfg.F)
    log(f"streamed: pinning {n_layers * cfg.E * nb / 1e9:.1f} GB of host experts")
    t0 = time.perf_counter()
    host, devs = [], []
    for l in range(n_layers):
        h = torch.empty((cfg.E, nb), dtype=torch.uint8, pin_memory=True)
        lw = gen.layer_weights(a.seed, l, cfg, experts_out=h.numpy())
        host.append(h)
        devs.append((moe.DeviceQMat(lw.router.codes, lw.router.meta, cfg.E, cfg.D, 8),
                     moe.DeviceBank.from_numpy(lw.shared[None, :], cfg.D, cfg.F_shared),
                     torch.from_numpy(gen.zipf_bias(a.seed, l, cfg.E, cfg.beta)).cuda()))
    log(f"host experts ready ({time.perf_counter() - t0:.1f} s)")
    slots = a.slots if a.slots > 0 else cfg.slots
    pool = moe.Pool(host, n_layers, slots, cfg.E, cfg.D, cfg.F)
    pool.set_policy(1 if a.pool_policy == "lru" else 0)
    xb = np.stack([gen.activations(a.seed, 2000 + l, 0, (n_tok + n_warm) * T, cfg.D, cfg.x_dtype)
                   for l in range(n_layers)])
    x_all = torch.from_numpy(xb.astype(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty(T, cfg.D, dtype=torch.float32, device="cuda")
    ws = moe.Workspace(T, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared)

    def token(t):
        for l in range(n_layers):
            router, shared, bias = devs[l]
            moe.moe_layer_forward(x_all[l, t * T:(t + 1) * T], router, cfg.k, None, shared, out,
                                  ws, logit_bias=bias, pool=pool, layer=l)

    for t in range(n_warm):  # warm the slots
        token(n_tok + t)
    torch.cuda.synchronize()
    pool.reset_stats()
    t0 = time.perf_counter()
    for t in range(n_tok):
        token(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st = pool.stats()
    # pinned host -> HBM copy peak for comparison
    src = host[0].reshape(-1)[: 256 << 20]
    dst = torch.empty(src.numel(), dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    peak = 4 * src.numel() / (time.perf_counter() - t1) / 1e9
    res = {"tokens": n_tok * T, "tokens_per_call": T, "layers": n_layers, "slots": slots,
           "policy": a.pool_policy, "s": el,
           "tokens_per_s": n_tok * T / el, "hit_rate": st["hits"] / max(1, st["lookups"]),
           "miss_MB_per_token": st["bytes_h2d"] / (n_tok * T) / 1e6,
           "h2d_GBps": st["bytes_h2d"] / el / 1e9, "pinned_copy_peak_GBps": peak, "beta": cfg.beta}
    log(f"streamed: {res}")
    pool.close()
    return res


def run_store(cfg, a, moe, torch):
    """The NVMe -> pinned-host tier: cold reads of expert blobs from a file on
    local storage by bounded-parallel pread (direct I/O) against mmap, then
    streamed decode with the pool's misses read from the file."""
    import tempfile
    n_layers = a.store_layers
    path = a.store_path or os.path.join(tempfile.gettempdir(), f"moe_experts_{os.getpid()}.bin")
    stride = gen.store_stride(cfg.D, cfg.F)
    nb = gen.blob_bytes(cfg.D, cfg.F)
    t0 = time.perf_counter()
    size = gen.write_expert_file(path, a.seed, n_layers, cfg)
    log(f"store: wrote {size / 1e9:.2f} GB ({n_layers} layers) to {path} in "
        f"{time.perf_counter() - t0:.1f} s")

    def drop_cache():
        fd = os.open(path, os.O_RDONLY)
        try:
            os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
        finally:
            os.close(fd)

    raw = torch.empty(16 * stride + 4096, dtype=torch.uint8, pin_memory=True)
    base = raw.data_ptr() + (-raw.data_ptr()) % 4096
    bufs = [base + i * stride for i in range(16)]
    rng = np.random.default_rng(a.seed + 1)
    res = {"config": "store", "layers": n_layers, "file_GB": size / 1e9,
           "expert_bytes": nb, "chunk_bytes": a.store_chunk}

    def cold(flags, threads, per_call, n_calls, chunk):
        drop_cache()
        st = moe.Store(path, n_layers, cfg.E, cfg.D, cfg.F, flags=flags, threads=threads)
        ms = []
        for _ in range(n_calls):
            layer = int(rng.integers(n_layers))
            ids = rng.choice(cfg.E, size=per_call, replace=False)
            t = time.perf_counter()
            st.read(layer, ids, bufs[:per_call], chunk)
            ms.append((time.perf_counter() - t) * 1e3)
        st.close()
        med = float(np.median(ms))
        return {"ms_per_call": med, "ms_per_expert": med / per_call,
                "GBps": per_call * nb / (med * 1e-3) / 1e9}

    qd = {}
    for threads in (1, 2, 4, 8, 16, 32):
        qd[str(threads)] = cold(moe.MOE_STORE_DIRECT, threads, 1, 24, a.store_chunk)
        log(f"store: pread direct, queue depth {threads}: {qd[str(threads)]}")
    res["pread_direct_one_expert_by_queue_depth"] = qd
    res["pread_direct_token_8_experts_qd32"] = cold(moe.MOE_STORE_DIRECT, 32, 8, 16, a.store_chunk)
    res["pread_buffered_one_expert_qd16"] = cold(0, 16, 1, 24, a.store_chunk)
    res["mmap_one_expert_1_thread"] = cold(moe.MOE_STORE_MMAP, 1, 1, 24, 0)
    res["mmap_one_expert_16_threads"] = cold(moe.MOE_STORE_MMAP, 16, 1, 24, a.store_chunk)
    log(f"store: {res}")

    # streamed decode, misses read from the file (pool staging -> HBM slots)
    slots = a.slots if a.slots > 0 else 16
    devs = []
    for l in range(n_layers):
        lw = gen.layer_weights(a.seed, l, cfg)
        devs.append((moe.DeviceQMat(lw.router.codes, lw.router.meta, cfg.E, cfg.D, 8),
                     moe.DeviceBank.from_numpy(lw.shared[None, :], cfg.D, cfg.F_shared),
                     torch.from_numpy(gen.zipf_bias(a.seed, l, cfg.E, gen.BETA_STACK)).cuda()))
    n_tok = a.stream_tokens
    xb = np.stack([gen.activations(a.seed, 2000 + l, 0, n_tok + 16, cfg.D, cfg.x_dtype)
                   for l in range(n_layers)])
    x_all = torch.from_numpy(xb.astype(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty(1, cfg.D, dtype=torch.float32, device="cuda")
    ws = moe.Workspace(1, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared)
    drop_cache()
    store = moe.Store(path, n_layers, cfg.E, cfg.D, cfg.F, flags=moe.MOE_STORE_DIRECT,
                      threads=a.store_threads)
    pool = moe.Pool.from_store(store, slots, chunk=a.store_chunk)

    def token(t):
        for l in range(n_layers):
            router, shared, bias = devs[l]
            moe.moe_layer_forward(x_all[l, t:t + 1], router, cfg.k, None, shared, out, ws,
                                  logit_bias=bias, pool=pool, layer=l)

    for t in range(16):
        token(n_tok + t)
    torch.cuda.synchronize()
    pool.reset_stats()
    s0 = store.stats()
    t0 = time.perf_counter()
    for t in range(n_tok):
        token(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    pst, s1 = pool.stats(), store.stats()
    read_s = (s1["ns"] - s0["ns"]) * 1e-9
    res["streamed_from_file"] = {
        "tokens": n_tok, "layers": n_layers, "slots": slots, "beta": gen.BETA_STACK,
        "layer_tokens_per_s": n_tok * n_layers / el, "us_per_layer_token": el * 1e6 / n_tok / n_layers,
        "hit_rate": pst["hits"] / max(1, pst["lookups"]),
        "miss_MB_per_layer_token": pst["bytes_h2d"] / (n_tok * n_layers) / 1e6,
        "store_read_GBps": (s1["bytes"] - s0["bytes"]) / max(read_s, 1e-9) / 1e9,
        "store_read_share_of_time": read_s / el, "store_threads": a.store_threads}
    log(f"store: streamed from file {res['streamed_from_file']}")
    pool.close()
    store.close()
    if not a.store_path:
        os.remove(path)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--config", default="decode",
                    choices=["decode", "prefill", "stack30", "streamed", "store"])
    ap.add_argument("--store-layers", type=int, default=4,
                    help="layers written to the expert file of the store workload")
    ap.add_argument("--store-path", default="",
                    help="expert file of the store workload (default: a temporary file)")
    ap.add_argument("--store-threads", type=int, default=32,
                    help="reads in flight of the store (queue depth)")
    ap.add_argument("--store-chunk", type=int, default=256 << 10,
                    help="bytes per pread piece of the store")
    ap.add_argument("--stream-tokens", type=int, default=64)
    ap.add_argument("--pool-policy", choices=["lfu", "lru"], default="lfu",
                    help="slot replacement of the streamed workload (lfu: the pages')")
    ap.add_argument("--slots", type=int, default=0,
                    help="HBM expert slots per layer for the streamed workload (default 16)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="tokens per step for decode / prefill (default: the workload's)")
    ap.add_argument("--block", action="store_true",
                    help="time the residual block (pre-norm, layer, post-norm and residual) "
                         "instead of the layer alone")
    ap.add_argument("--beta", type=float, default=None,
                    help="Zipf skew of the router-logit bias (default: the workload's own)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph-steps", type=int, default=64)
    ap.add_argument("--regions", type=int, default=5,
                    help="timed regions of --steps steps each; the median is reported")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device copy (counter calibration)")
    ap.add_argument("--tune", action="append", default=[],
                    help="launch-shape knob key=value (moe_set_tuning), repeatable")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_mixture_experts_moe_amd import moe

    torch.cuda.set_device(0)
    for kv in a.tune:
        key, val = kv.split("=")
        moe.moe_set_tuning(key, int(val))
    if a.config == "store":
        res = run_store(gen.CONFIGS["streamed"], a, moe, torch)
        print(json.dumps(res), flush=True)
        return
    cfg = gen.CONFIGS[a.config]
    if a.beta is not None:
        import dataclasses
        cfg = dataclasses.replace(cfg, beta=a.beta)
    if a.config in ("stack30", "streamed"):
        res = (run_stack if a.config == "stack30" else run_streamed)(cfg, a, moe, torch)
        print(json.dumps({"config": a.config, **res}), flush=True)
        return
    n_layers = cfg.layers
    T = a.tokens if a.tokens > 0 else cfg.T
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
    ws = moe.Workspace(T, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared, block=a.block)
    if a.block:
        xb = np.concatenate([gen.residual_stream(a.seed, 1000 + i, 0, T, cfg.D, cfg.x_dtype)
                             for i in range(n_x)])
        x_all = torch.from_numpy(xb.astype(np.int16)).cuda().view(torch.bfloat16).reshape(
            n_x, T, cfg.D)
        norms = [tuple(torch.from_numpy(w).cuda() for w in gen.norm_weights(a.seed, l, cfg.D))
                 for l in range(n_layers)]

    def step(i):
        router, routed, shared, bias = layers[i % n_layers]
        if a.block:
            w_pre, w_post = norms[i % n_layers]
            moe.moe_block_forward(x_all[i % n_x], w_pre, w_post, 1e-6, router, cfg.k, routed,
                                  shared, out[i % n_x], ws, logit_bias=bias)
            return
        moe.moe_layer_forward(x_all[i % n_x], router, cfg.k, routed, shared, out[i % n_x], ws,
                              logit_bias=bias)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(G):  # eager pass (also loads the kernels)
            step(i)
    torch.cuda.synchronize()
    graphs = {}

    def graph_of(n):
        # one graph of n consecutive steps, captured once
        if n not in graphs:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for i in range(n):
                    step(i)
            torch.cuda.synchronize()
            graphs[n] = gr
        return graphs[n]

    def run(n):
        # exactly n steps: full graphs of G steps, then one of the remainder
        full, rem = divmod(n, G)
        gf = graph_of(G) if full else None
        gr = graph_of(rem) if rem else None
        with torch.cuda.stream(stream):
            for _ in range(full):
                gf.replay()
            if gr is not None:
                gr.replay()

    steps = max(1, a.steps)
    graph_of(G)
    graph_of(steps % G) if steps % G else None
    graph_of(a.warmup % G) if a.warmup % G else None
    run(a.warmup)
    torch.cuda.synchronize()
    # the median of several timed regions of exactly `steps` steps each
    region_ms = []
    for _ in range(max(1, a.regions)):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        run(steps)
        ev1.record(stream)
        torch.cuda.synchronize()
        region_ms.append(ev0.elapsed_time(ev1))
    ms = float(np.median(region_ms))
    ms_step = ms / steps
    tokens_per_s = steps * T / (ms / 1e3)
    step_bytes = gen.algorithmic_decode_bytes(cfg) * T if T == 1 else None
    gbps = step_bytes / (ms_step / 1e3) / 1e9 if step_bytes else None
    log(f"{steps} steps in {ms:.2f} ms: {ms_step * 1e3:.2f} us/step, {tokens_per_s:,.0f} tokens/s"
        + (f", {gbps:,.0f} GB/s" if gbps else ""))

    # duration of the dominant kernel.  A decode step on the one-launch path
    # is exactly one launch of the layer kernel, so its average duration is
    # the timed region's (HIP events on the stream the graphs replay on) per
    # step.  Otherwise (the expert phase of a prefill chunk, or of a decode
    # step on the router + expert-phase path) the library records events
    # around that phase's launches on the same stream, in eager steps.
    layer_path = T == 1 and "layer=0" not in a.tune and not a.block
    tune = dict(kv.split("=") for kv in a.tune)
    grouped = T >= int(tune.get("prefill_min_t", 8))  # the library's default crossover
    if layer_path or (T > 1 and not grouped) or a.block:
        # one launch per step, or (2 to 7 tokens) the router kernel and the
        # few-token expert kernels, timed as the whole step
        k_us = ms_step * 1e3
    else:
        n_prof = min(512, steps)
        with moe.ProfileEvents(n_prof) as pe, torch.cuda.stream(stream):
            for i in range(n_prof):
                step(i)
            torch.cuda.synchronize()
            kms = pe.elapsed_ms(n_prof)
        k_us = 1e3 * float(np.mean(kms))
    if a.block:
        # the layer's bytes plus the block's own: x read by both norms, the
        # two weight vectors
        k_bytes = (gen.algorithmic_decode_bytes(cfg) + cfg.D * 2 + 2 * cfg.D * 4
                   if T == 1 else None)
        k_name = "whole residual block step (pre-norm, layer, post-norm and residual)"
        traffic = None
    elif layer_path:
        k_bytes = gen.algorithmic_decode_bytes(cfg)
        k_name = ("decode_layer_kernel (router, top-8, gate/up, down and combine of the 8 "
                  "routed and the shared expert in one launch)")
        traffic = stored_traffic("decode_layer_traffic.json")
    elif T == 1:
        k_bytes = gen.algorithmic_decode_bytes(cfg) - gen.codes_bytes(cfg.E, cfg.D, 8) \
            - gen.meta_bytes(cfg.E, cfg.D)
        k_name = "experts_fused_kernel (gate/up + down + combine of the 8 routed and the shared expert)"
        traffic = stored_traffic("decode_expert_phase_traffic.json")
    else:
        # the expert phase of a chunk reads every selected expert's blob once
        # (experts chosen by several tokens serve all their rows from one
        # read), the shared expert, the activation pairs and the outputs
        ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
        gates = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
        uniq = []
        for i in range(n_x):
            router, routed, shared, bias = layers[i % n_layers]
            moe.moe_route(x_all[i], router, cfg.k, ids, gates, ws, bias)
            torch.cuda.synchronize()
            uniq.append(len(np.unique(ids.cpu().numpy())))
        k_bytes = (float(np.mean(uniq)) * gen.blob_bytes(cfg.D, cfg.F)
                   + (gen.blob_bytes(cfg.D, cfg.F_shared) if cfg.F_shared else 0)
                   + T * cfg.D * 2 + T * cfg.D * 4)
        if not grouped:
            k_bytes += gen.codes_bytes(cfg.E, cfg.D, 8) + gen.meta_bytes(cfg.E, cfg.D)
            if T <= 2 and tune.get("layer", "1") != "0":
                how = "one launch of the layer kernel"
            elif tune.get("mid", "0") != "0" and T <= int(tune.get("mid_max_t", 7)):
                how = ("router kernel and the batched-decode expert kernels (each distinct "
                       "expert and the shared expert read once)")
            else:
                how = "router kernel and the few-token expert kernels"
            k_name = f"whole step of {T} tokens: {how} ({np.mean(uniq):.1f} distinct experts)"
        else:
            k_name = (f"grouped prefill expert kernels (gate/up, down, combine; "
                      f"{np.mean(uniq):.1f} distinct experts per chunk)")
        traffic = None
    k_gbps = k_bytes / (k_us * 1e-6) / 1e9 if k_bytes else None
    log(f"timed kernel: {k_us:.2f} us per launch" + (f", {k_gbps:,.0f} GB/s" if k_gbps else ""))

    if a.calibrate_copy:
        # a plain copy of known size, for scaling the HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # the chip's streaming read rate, measured: a read of a 4 GiB buffer (far
    # beyond the Infinity Cache), best of five
    probe = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    read_gbps = 0.0
    with torch.cuda.stream(stream):
        for i in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            moe.moe_read_probe(probe, sink, 8192, stream)
            e1.record(stream)
            e1.synchronize()
            if i:
                read_gbps = max(read_gbps, probe.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del probe
    log(f"streaming read of 4 GiB: {read_gbps:,.0f} GB/s")

    cpu = None
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(cfg, a.seed, a.cpu_seconds, block=a.block)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "timed_regions_ms": [round(v, 4) for v in region_ms],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations, int4/int8 weights, fp32 accumulate",
        "data": "synthetic (seeded weights and activations)",
        "config": {"workload": f"{cfg.name}: "
                               + ("residual block (RMSNorm, layer, RMSNorm, residual) around "
                                  if a.block else "")
                               + "one Gemma-4-26B-A4B-shaped MoE layer, "
                               f"{T} token(s) per step, d_model {cfg.D}, {cfg.E} experts of "
                               f"GLU width {cfg.F} (4-bit, group 64), top-{cfg.k}, shared expert "
                               f"{cfg.F_shared}, 8-bit router; {n_layers} seeded layer replicas "
                               f"rotated" + (f", Zipf-biased routing (beta {cfg.beta})"
                                             if cfg.beta else ""),
                   "tokens_per_step": T, "layers_rotated": n_layers,
                   "parallelism": "single GPU"},
        "hbm_GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": k_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": k_gbps / HBM_PEAK_GBPS if k_gbps else None, "traffic": traffic,
                     "measured_read_peak": read_gbps,
                     "frac_of_measured_read_peak": (k_gbps / read_gbps
                                                    if k_gbps and read_gbps else None),
                     "kernel": k_name, "us_per_launch": k_us,
                     "algorithmic_bytes_per_launch": k_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
