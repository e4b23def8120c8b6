"""GPU parity of the residual block (moe_block_forward) against the oracle.

The block is RMSNorm(x) -> layer -> RMSNorm -> + x.  Its two checks:

* the layer's input u (the pre-norm, rounded to 16 bits in fp32 as the kernel
  rounds it) bit-exact against the oracle's float64 pre-norm rounded through
  fp32, except where the float64 value lies within a relative 4e-6 of a
  rounding boundary: there either neighbour is accepted.  The kernel's fp32
  value is within about 1e-6 relative of the exact one (a sum of squares
  over at most 32 terms per thread, a 6-level wave tree and 4 waves, then a
  correctly rounded divide, square root, reciprocal and three products), so
  4e-6 leaves a margin of four.
* the block output against the oracle fed the GPU's u and ids.  The layer's
  own bars (relative L2 1e-3, max-abs 2e-2 on y) carry through the post-norm
  as |1 + w_post| / rms(y) * (2e-2 + 2e-3 |y|) per element: the norm of y
  moves by at most the relative L2 error, the rest is the element's own
  error, both scaled by the norm; plus 1e-5 of the element for the fp32
  residual add.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import gen
from tests._helpers import MAX_ABS, REL_L2, check_ids, rel_l2
from tests.test_gpu_parity import TORCH_X, dev_layer, oracle_rows

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("quantized_mixture_experts_moe_amd.moe")

EPS = O.NORM_EPS
U_BOUNDARY = 4e-6


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _dev(bits, dtype):
    return torch.from_numpy(bits.astype(np.int16)).cuda().view(TORCH_X[dtype])


def _round16(v, dtype):
    if dtype == "bf16":
        return O.round_to_bf16(v)
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float16).view(np.uint16)


def _block_gpu(L, xb, w_pre, w_post, bias=None, out_dtype=torch.float32, in_place=False):
    cfg = L.cfg
    T = xb.shape[0]
    ws = moe.Workspace(T, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared, block=True)
    x = _dev(xb, cfg.x_dtype)
    out = x if in_place else torch.empty(T, cfg.D, dtype=out_dtype, device="cuda")
    u = torch.empty(T, cfg.D, dtype=TORCH_X[cfg.x_dtype], device="cuda")
    ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    bias_d = torch.from_numpy(bias).cuda() if bias is not None else None
    moe.moe_block_forward(x, torch.from_numpy(w_pre).cuda(), torch.from_numpy(w_post).cuda(), EPS,
                          L.router, cfg.k, L.routed, L.shared, out, ws, logit_bias=bias_d,
                          u_out=None if in_place else u, ids_out=ids)
    torch.cuda.synchronize()
    assert ws.timeouts() == 0
    u_bits = u.view(torch.int16).cpu().numpy().view(np.uint16)
    return out, u_bits, ids.cpu().numpy()


def _check_u(xf, w_pre, u_bits, dtype):
    v = O.rms_norm(xf, w_pre, EPS)
    lo = _round16(v * (1 - U_BOUNDARY), dtype)
    hi = _round16(v * (1 + U_BOUNDARY), dtype)
    sure = lo == hi
    assert np.array_equal(u_bits[sure], lo[sure])
    assert np.all((u_bits == lo) | (u_bits == hi))
    print(f"    u: {np.count_nonzero(~sure)} of {u_bits.size} near a rounding boundary",
          flush=True)
    # a value falls within the band about a boundary with probability about
    # 2 U_BOUNDARY / (relative spacing), spacing 2^-8 (bf16) or 2^-11 (fp16)
    frac = 2 * U_BOUNDARY * (2.0 ** (8 if dtype == "bf16" else 11))
    assert np.count_nonzero(~sure) < 8 + 2 * frac * u_bits.size


def _check_out(xf, y_ref, w_post, got):
    ref = xf + O.rms_norm(y_ref, w_post, EPS)
    inv = 1.0 / np.sqrt(np.mean(y_ref ** 2, axis=1, keepdims=True) + EPS)
    bound = (np.abs(1.0 + w_post.astype(np.float64)) * inv * (MAX_ABS + 2 * REL_L2 * np.abs(y_ref))
             + 1e-5 * np.abs(ref))
    err = np.abs(got - ref)
    r = rel_l2(got - xf, ref - xf)
    print(f"    block rel_l2={r:.2e} worst err/bound={np.max(err / bound):.3f}", flush=True)
    assert r < REL_L2
    assert np.all(err < bound)


@pytest.mark.parametrize("name,T,beta,rows", [("tiny", 5, 0.0, None), ("decode", 1, 0.0, None),
                                              ("decode", 4, 6.5, None),
                                              ("decode", 128, 1.5, [0, 1, 63, 64, 100, 127])])
def test_block_forward_parity(name, T, beta, rows):
    """Decode (one token: the one-launch layer kernel), a few-token batch and
    a 128-token prefill chunk (the matrix-core path; u on every row, the
    output on sampled rows), residual rows of norms from 1/4 to 16."""
    _case(f"block_forward {name} T={T} beta={beta}")
    L = dev_layer(name)
    cfg = L.cfg
    xb = gen.residual_stream(3, 0, 0, T, cfg.D, cfg.x_dtype)
    w_pre, w_post = gen.norm_weights(0, 0, cfg.D)
    bias = gen.zipf_bias(0, 0, cfg.E, beta) if beta else None
    out, u_bits, ids = _block_gpu(L, xb, w_pre, w_post, bias)
    xf = O.activations_to_float(xb, cfg.x_dtype)
    _check_u(xf, w_pre, u_bits, cfg.x_dtype)
    rows = list(range(T)) if rows is None else rows
    uf = O.activations_to_float(u_bits[rows], cfg.x_dtype)
    y_ref, logits = oracle_rows(L, uf, ids[rows], bias)
    check_ids(logits, ids[rows], cfg.k)
    _check_out(xf[rows], y_ref, w_post, out.cpu().numpy()[rows])


def test_block_forward_end_to_end_oracle():
    """The small layer against the oracle's own block (pre-norm, rounding,
    layer, post-norm, residual), ids compared gap-aware, with a zero row (u
    is zero, the output is the norm of the layer's response to zero)."""
    _case("block_forward tiny T=6, oracle block_forward, zero row")
    L = dev_layer("tiny")
    cfg = L.cfg
    xb = gen.residual_stream(5, 0, 0, 6, cfg.D, cfg.x_dtype)
    xb[2] = 0
    w_pre, w_post = gen.norm_weights(1, 0, cfg.D)
    out, u_bits, ids = _block_gpu(L, xb, w_pre, w_post)
    xf = O.activations_to_float(xb, cfg.x_dtype)
    assert not np.any(u_bits[2] & 0x7FFF)
    ref = O.block_forward(xf, L.lw, cfg.k, w_pre, w_post, EPS, x_dtype=cfg.x_dtype,
                          u=O.activations_to_float(u_bits, cfg.x_dtype))
    check_ids(ref["logits"], ids, cfg.k)
    ref = O.block_forward(xf, L.lw, cfg.k, w_pre, w_post, EPS, x_dtype=cfg.x_dtype,
                          u=O.activations_to_float(u_bits, cfg.x_dtype), ids=ids)
    _check_out(xf, ref["moe"], w_post, out.cpu().numpy())


@pytest.mark.parametrize("T", [1, 3, 128])
def test_block_forward_in_place_and_out_dtypes(T):
    """out == x (the residual stream updated in place) gives the same bits as
    a separate bf16 output, which is the fp32 output rounded to nearest even."""
    _case(f"block_forward in place T={T}")
    L = dev_layer("decode")
    cfg = L.cfg
    xb = gen.residual_stream(7, 0, 0, T, cfg.D, cfg.x_dtype)
    w_pre, w_post = gen.norm_weights(0, 0, cfg.D)
    bias = gen.zipf_bias(0, 0, cfg.E, 1.5) if T == 128 else None
    o32, _, i32 = _block_gpu(L, xb, w_pre, w_post, bias)
    o16, _, i16 = _block_gpu(L, xb, w_pre, w_post, bias, out_dtype=torch.bfloat16)
    oin, _, iin = _block_gpu(L, xb, w_pre, w_post, bias, in_place=True)
    assert np.array_equal(i32, i16) and np.array_equal(i32, iin)
    b16 = o16.view(torch.int16).cpu().numpy()
    assert np.array_equal(b16, oin.view(torch.int16).cpu().numpy())
    assert np.array_equal(b16.view(np.uint16), O.round_to_bf16(o32.cpu().numpy()))


def test_block_forward_repeatable():
    _case("block_forward bitwise repeatable T=1")
    L = dev_layer("decode")
    cfg = L.cfg
    xb = gen.residual_stream(9, 0, 0, 1, cfg.D, cfg.x_dtype)
    w_pre, w_post = gen.norm_weights(0, 0, cfg.D)
    a, _, _ = _block_gpu(L, xb, w_pre, w_post)
    b, _, _ = _block_gpu(L, xb, w_pre, w_post)
    assert torch.equal(a, b)


def _set_fused(v):
    moe.moe_set_tuning("block_fused", v)


@pytest.mark.parametrize("name,T,in_place", [("decode", 1, False), ("decode", 1, True),
                                             ("decode", 2, False), ("decode", 2, True),
                                             ("decode", 4, True), ("tiny", 3, False),
                                             ("tiny", 4, True)])
def test_block_fused_launch_equals_separate_kernels(name, T, in_place):
    """The one-launch decode layer with both norms inside gives the same bits
    as the three-step path (pre-norm kernel, layer, post-norm kernel): the
    layer's input u, the ids and the block output, over repeated calls (the
    per-token counters return to zero)."""
    _case(f"block fused vs separate {name} T={T} in_place={in_place}")
    L = dev_layer(name)
    cfg = L.cfg
    xb = gen.residual_stream(11, 0, T, T, cfg.D, cfg.x_dtype)
    w_pre, w_post = gen.norm_weights(2, 0, cfg.D)
    odt = TORCH_X[cfg.x_dtype] if in_place else torch.float32
    try:
        _set_fused(0)
        ref, ref_u, ref_ids = _block_gpu(L, xb, w_pre, w_post, out_dtype=odt, in_place=in_place)
        _set_fused(1)
        for _ in range(3):
            got, got_u, got_ids = _block_gpu(L, xb, w_pre, w_post, out_dtype=odt,
                                             in_place=in_place)
            assert np.array_equal(got_ids, ref_ids)
            if not in_place:
                assert np.array_equal(got_u, ref_u)
            assert torch.equal(got.view(torch.int16) if odt != torch.float32 else got,
                               ref.view(torch.int16) if odt != torch.float32 else ref)
    finally:
        _set_fused(1)


@pytest.mark.parametrize("T", [2, 3])
def test_block_fused_with_one_router_block_per_group(T):
    """Four experts: a token group has one router block, which then does the
    post-norm of both its tokens; fused equals the separate kernels and the
    oracle."""
    _case(f"block fused, E=4 (one router block per token group), T={T}")
    from tests.test_gpu_parity import DevLayer
    cfg = gen.MoEConfig("e4", D=256, E=4, F=128, F_shared=256, k=2, T=T, x_dtype="fp16")
    L = DevLayer(cfg, seed=3)
    xb = gen.residual_stream(13, 0, T, T, cfg.D, cfg.x_dtype)
    w_pre, w_post = gen.norm_weights(4, 0, cfg.D)
    try:
        _set_fused(0)
        ref, ref_u, ref_ids = _block_gpu(L, xb, w_pre, w_post)
        _set_fused(1)
        got, got_u, got_ids = _block_gpu(L, xb, w_pre, w_post)
    finally:
        _set_fused(1)
    assert np.array_equal(got_ids, ref_ids) and np.array_equal(got_u, ref_u)
    assert torch.equal(got, ref)
    xf = O.activations_to_float(xb, cfg.x_dtype)
    out = O.block_forward(xf, L.lw, cfg.k, w_pre, w_post, EPS, x_dtype=cfg.x_dtype,
                          u=O.activations_to_float(got_u, cfg.x_dtype), ids=got_ids)
    _check_out(xf, out["moe"], w_post, got.cpu().numpy())


def test_block_forward_streamed_equals_resident():
    """The block over a slot pool (pre-norm kernel, the layer in two launches
    with the experts streamed into 4 HBM slots, post-norm kernel) gives the
    bits of the resident block (both norms inside the one-launch layer)."""
    _case("block_forward pooled vs resident (tiny, 4 slots, 12 tokens)")
    L = dev_layer("tiny", seed=3)
    cfg = L.cfg
    host = [torch.from_numpy(L.lw.experts.copy()).pin_memory()]
    pool = moe.Pool(host, 1, 4, cfg.E, cfg.D, cfg.F)
    ws = moe.Workspace(1, cfg.k, cfg.E, cfg.D, cfg.F, cfg.F_shared, block=True)
    w_pre, w_post = gen.norm_weights(5, 0, cfg.D)
    wp, wq = torch.from_numpy(w_pre).cuda(), torch.from_numpy(w_post).cuda()
    bias = torch.from_numpy(gen.zipf_bias(3, 0, cfg.E, 4.0)).cuda()
    try:
        for tok in range(12):
            xb = gen.residual_stream(17, 0, tok, 1, cfg.D, cfg.x_dtype)
            x = _dev(xb, cfg.x_dtype)
            o_s = torch.empty(1, cfg.D, dtype=torch.float32, device="cuda")
            o_r = torch.empty_like(o_s)
            moe.moe_block_forward(x, wp, wq, EPS, L.router, cfg.k, None, L.shared, o_s, ws,
                                  logit_bias=bias, pool=pool, layer=0)
            moe.moe_block_forward(x, wp, wq, EPS, L.router, cfg.k, L.routed, L.shared, o_r, ws,
                                  logit_bias=bias)
            torch.cuda.synchronize()
            assert torch.equal(o_s, o_r), tok
        assert ws.timeouts() == 0
        assert pool.stats()["misses"] > 0
    finally:
        pool.close()
