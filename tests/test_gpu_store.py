"""Streamed experts from a file on local storage (the expert store): the
pool reads each call's missing experts with parallel pread into page-locked
staging and copies them into its HBM slots.  Output bitwise the resident
output, hits and misses those of the oracle's LFU model, and the store read
exactly the missing blobs."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import gen
from tests._helpers import MAX_ABS, REL_L2, max_abs, rel_l2

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("quantized_mixture_experts_moe_amd.moe")


@pytest.mark.parametrize("name,layers,slots,flags,path", [
    ("tiny", 2, 4, 1, "layer"), ("tiny", 2, 4, 0, "three"), ("decode", 2, 16, 1, "layer"),
    ("decode", 1, 16, 2, "layer")])
def test_pool_from_store_equals_resident(tmp_path, name, layers, slots, flags, path):
    cfg = gen.CONFIGS[name]
    print(f"[case] store pool {name} layers={layers} slots={slots} flags={flags} {path}", flush=True)
    file = str(tmp_path / "experts.bin")
    gen.write_expert_file(file, 0, layers, cfg)
    store = moe.Store(file, layers, cfg.E, cfg.D, cfg.F, flags=flags, threads=16)
    pool = moe.Pool.from_store(store, slots, chunk=256 << 10)
    devs = []
    for l in range(layers):
        lw = gen.layer_weights(0, l, cfg)
        devs.append((lw, moe.DeviceQMat(lw.router.codes, lw.router.meta, cfg.E, cfg.D, 8),
                     moe.DeviceBank.from_numpy(lw.experts, cfg.D, cfg.F),
                     moe.DeviceBank.from_numpy(lw.shared[None, :], cfg.D, cfg.F_shared)))
    ws = moe.Workspace(1, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared)
    if path == "three":
        moe.moe_set_tuning("layer", 0)
        moe.moe_set_tuning("fused", 0)
    try:
        models = [O.LFUCache(slots, cfg.E) for _ in range(layers)]
        misses = 0
        tokens = 6
        for tok in range(tokens):
            for l, (lw, router, routed, shared) in enumerate(devs):
                xb = gen.activations(9, l, tok, 1, cfg.D, cfg.x_dtype)
                tdt = torch.float16 if cfg.x_dtype == "fp16" else torch.bfloat16
                x = torch.from_numpy(xb.astype(np.int16)).cuda().view(tdt)
                bias_np = gen.zipf_bias(0, l, cfg.E, 4.0)
                bias = torch.from_numpy(bias_np).cuda()
                o_s = torch.empty(1, cfg.D, dtype=torch.float32, device="cuda")
                o_r = torch.empty_like(o_s)
                ids = torch.empty(1, cfg.k, dtype=torch.int32, device="cuda")
                moe.moe_layer_forward(x, router, cfg.k, None, shared, o_s, ws, logit_bias=bias,
                                      pool=pool, layer=l, ids_out=ids)
                moe.moe_layer_forward(x, router, cfg.k, routed, shared, o_r, ws, logit_bias=bias)
                torch.cuda.synchronize()
                assert torch.equal(o_s, o_r), (tok, l)
                got_ids = ids.cpu().numpy()
                ev = models[l].access(got_ids[0])
                misses += sum(1 for e in ev if not e[2])
                if tok == tokens - 1 and l == 0:
                    xf = O.activations_to_float(xb, cfg.x_dtype)
                    ref = O.layer_forward(xf, lw, cfg.k, bias_np, ids=got_ids)
                    got = o_s.cpu().numpy()
                    assert rel_l2(got, ref["out"]) < REL_L2 and max_abs(got, ref["out"]) < MAX_ABS
        st = pool.stats()
        assert st["misses"] == misses and st["lookups"] == tokens * layers * cfg.k
        assert store.stats()["blobs"] == misses
        assert ws.timeouts() == 0
    finally:
        moe.moe_set_tuning("layer", 1)
        moe.moe_set_tuning("fused", 1)
        pool.close()
        store.close()


def test_store_pool_prefill_chunk_in_expert_batches(tmp_path):
    """A 128-token chunk of the Gemma-shaped layer through a 16-slot pool fed
    from the expert file: its experts run in batches of 16, the staging
    buffers of a slot index are reused from batch to batch.  Output bitwise
    the resident chunk's, and the store read each distinct expert once."""
    cfg = gen.CONFIGS["prefill"]
    print("[case] store pool, prefill chunk T=128, 16 slots (expert batches)", flush=True)
    file = str(tmp_path / "experts.bin")
    gen.write_expert_file(file, 0, 1, cfg)
    store = moe.Store(file, 1, cfg.E, cfg.D, cfg.F, flags=1, threads=16)
    pool = moe.Pool.from_store(store, 16, chunk=256 << 10)
    lw = gen.layer_weights(0, 0, cfg)
    router = moe.DeviceQMat(lw.router.codes, lw.router.meta, cfg.E, cfg.D, 8)
    routed = moe.DeviceBank.from_numpy(lw.experts, cfg.D, cfg.F)
    shared = moe.DeviceBank.from_numpy(lw.shared[None, :], cfg.D, cfg.F_shared)
    ws = moe.Workspace(cfg.T, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared)
    bias = torch.from_numpy(gen.zipf_bias(0, 0, cfg.E, cfg.beta)).cuda()
    try:
        xb = gen.activations(0, 0, 0, cfg.T, cfg.D, cfg.x_dtype)
        x = torch.from_numpy(xb.astype(np.int16)).cuda().view(torch.bfloat16)
        o_s = torch.empty(cfg.T, cfg.D, dtype=torch.float32, device="cuda")
        o_r = torch.empty_like(o_s)
        ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
        moe.moe_layer_forward(x, router, cfg.k, None, shared, o_s, ws, logit_bias=bias,
                              pool=pool, layer=0, ids_out=ids)
        moe.moe_layer_forward(x, router, cfg.k, routed, shared, o_r, ws, logit_bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_r)
        distinct = len(np.unique(ids.cpu().numpy()))
        assert distinct > 16
        assert pool.stats()["misses"] == distinct and store.stats()["blobs"] == distinct
        assert ws.timeouts() == 0
    finally:
        pool.close()
        store.close()


def test_read_probe_reads_every_word():
    """The streaming read probe: the words it writes (the xor of each
    workgroup's 16-byte loads) xor to the xor of the whole buffer."""
    print("[case] read probe", flush=True)
    n = (64 << 20) + 16 * 1000  # a tail past the unrolled part
    host = np.random.default_rng(3).integers(0, 2**32, size=n // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    for blocks in (1, 300, 8192):
        sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
        moe.moe_read_probe(buf, sink, blocks)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), blocks
