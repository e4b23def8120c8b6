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
