"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test fixes a part of the oracle against a hand-built input, a closed
form, a library routine the case reduces to, an independent brute-force
evaluation, or a figure the pages print.  The mutation tests at the end plant
plausible mistakes in a copy of the oracle and check that a pin catches them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from synthetic import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class _Layer:
    def __init__(self, router, experts, shared, D, F, F_shared):
        self.router, self.experts, self.shared = router, experts, shared
        self.D, self.F, self.F_shared = D, F, F_shared


def _tiny_layer(seed=0, D=256, E=16, F=128, F_shared=256, layer=0):
    cfg = gen.MoEConfig("t", D=D, E=E, F=F, F_shared=F_shared, k=4, T=4, x_dtype="fp16")
    return gen.layer_weights(seed, layer, cfg)


# ---------------------------------------------------------------- storage format
def test_unpack_handbuilt_4bit_words():
    # R = 2 rows, C = 64 columns, 4-bit: chunks of 32 columns, chunk-major.
    raw = np.zeros(2 * 64 // 2, dtype=np.uint8)
    raw[0:4] = np.frombuffer(np.uint32(0x76543210).tobytes(), np.uint8)  # chunk (cc0, r0)
    raw[16] = 0x9A                     # chunk (cc0, r1): col 0 -> 0xA, col 1 -> 0x9
    raw[32 + 15] = 0xF0                # chunk (cc1, r0): col 62 -> 0x0, col 63 -> 0xF
    raw[48 + 8] = 0x05                 # chunk (cc1, r1): col 48 -> 5
    q = O.unpack_codes(raw, 2, 64, 4)
    assert list(q[0, :8]) == [0, 1, 2, 3, 4, 5, 6, 7]
    assert q[1, 0] == 10 and q[1, 1] == 9
    assert q[0, 62] == 0 and q[0, 63] == 15
    assert q[1, 48] == 5
    assert q.sum() == 28 + 19 + 15 + 5


def test_unpack_handbuilt_8bit_words():
    raw = np.zeros(3 * 64, dtype=np.uint8)   # R = 3, C = 64, 16 columns per chunk
    raw[(1 * 3 + 2) * 16 + 5] = 200          # chunk (cc1, r2), position 5 -> col 21
    raw[(3 * 3 + 0) * 16 + 15] = 7           # chunk (cc3, r0), position 15 -> col 63
    q = O.unpack_codes(raw, 3, 64, 8)
    assert q[2, 21] == 200 and q[0, 63] == 7 and q.sum() == 207


def test_pack_unpack_roundtrip_random():
    rng = np.random.default_rng(3)
    for bits, (R, C) in ((4, (5, 128)), (8, (7, 192)), (4, (64, 2816 // 11))):
        if C % 64:
            continue
        codes = rng.integers(0, 1 << bits, size=(R, C))
        packed = gen.pack_codes(codes, bits)
        assert np.array_equal(O.unpack_codes(packed, R, C, bits), codes)


def test_meta_handbuilt():
    # scale 1.0 (0x3C00), bias -2.0 (0xC000) for group 0 of row 0; row 1 scale 0.5.
    meta = np.array([0x3C00 | (0xC000 << 16), 0x3800, 0x0, 0x0], dtype=np.uint32)
    s, b = O.unpack_meta(meta, 2, 128)  # layout [group][row]
    assert float(s[0, 0]) == 1.0 and float(b[0, 0]) == -2.0
    assert float(s[1, 0]) == 0.5 and float(b[1, 0]) == 0.0
    assert float(s[0, 1]) == 0.0


def test_onehot_selects_one_dequantised_column():
    # 4-bit W[3, 128]: code 7 at (1, 70) with group-1 scale 0.5, bias -2.0.
    codes = np.zeros((3, 128), dtype=np.int64)
    codes[1, 70] = 7
    scale = np.full((3, 2), 0.25, np.float16)
    bias = np.zeros((3, 2), np.float16)
    scale[1, 1], bias[1, 1] = 0.5, -2.0
    rt = gen.RouterQ(gen.pack_codes(codes, 4), gen.pack_meta(scale, bias), 3, 128, 4)
    x = np.zeros((1, 128))
    x[0, 70] = 1.0
    l = O.router_logits(x, rt)
    assert l[0, 1] == 1.5          # 0.5 * 7 - 2
    assert l[0, 0] == 0.0 and l[0, 2] == 0.0
    x[0, 70], x[0, 3] = 0.0, 1.0   # column 3 is in group 0: 0.25 * 0 + 0
    assert np.all(O.router_logits(x, rt) == 0.0)


def test_constant_codes_closed_form():
    # every code 3, scale 0.25, bias 0.5: W x = 1.25 * sum(x) on every row
    codes = np.full((4, 192), 3)
    rt = gen.RouterQ(gen.pack_codes(codes, 8), gen.pack_meta(np.full((4, 3), 0.25, np.float16),
                                                             np.full((4, 3), 0.5, np.float16)), 4, 192, 8)
    x = np.arange(192, dtype=np.float64)[None, :] / 8.0
    l = O.router_logits(x, rt)
    assert np.all(l == 1.25 * (191 * 192 / 2) / 8.0)


def test_quantise_dequantise_error_bound():
    # a min/max affine quantiser (MLX-style) reproduces weights within scale/2
    rng = np.random.default_rng(5)
    W = rng.standard_normal((6, 128))
    g = W.reshape(6, 2, 64)
    lo, hi = g.min(axis=2), g.max(axis=2)
    scale = ((hi - lo) / 15).astype(np.float16)
    bias = lo.astype(np.float16)
    q = np.clip(np.rint((g - bias[..., None].astype(np.float64)) / scale[..., None].astype(np.float64)), 0, 15)
    rt = gen.RouterQ(gen.pack_codes(q.reshape(6, 128).astype(np.int64), 4),
                     gen.pack_meta(scale, bias), 6, 128, 4)
    Wd = O.dequantize(rt.codes, rt.meta, 6, 128, 4)
    err = np.abs(Wd - W).reshape(6, 2, 64).max(axis=2)
    # bound: half a step plus the fp16 rounding of the scale and bias
    bound = scale.astype(np.float64) / 2 + 15 * np.abs(scale.astype(np.float64) - (hi - lo) / 15) \
        + np.abs(bias.astype(np.float64) - lo)
    assert np.all(err <= bound + 1e-12)


# ---------------------------------------------------------------- activation and routing
def _golden_gelu():
    rows = []
    with open(os.path.join(GOLDEN, "gelu_tanh_points.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


def test_gelu_tanh_golden_points():
    for x, tanh_form, erf_form in _golden_gelu():
        assert float(O.gelu_tanh(np.float64(x))) == pytest.approx(tanh_form, abs=1e-15)
        if x != 0.0:
            assert abs(tanh_form - erf_form) > 1e-5


def test_x_zero():
    lw = _tiny_layer()
    out = O.layer_forward(np.zeros((2, 256)), lw, 4)
    assert np.all(out["logits"] == 0.0)
    assert np.array_equal(out["ids"], np.tile(np.arange(4), (2, 1)))
    assert np.all(out["gates"] == 0.25)
    assert np.all(out["out"] == 0.0)


def test_k_equals_E_is_plain_softmax():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((5, 16)) * 3
    ids, gates = O.select_topk(logits, 16)
    for t in range(5):
        order = np.argsort(-logits[t].astype(np.float32), kind="stable")
        assert np.array_equal(ids[t], order)
        np.testing.assert_allclose(gates[t], scipy.special.softmax(logits[t])[order], rtol=1e-13)


def test_topk_ties_go_to_lower_index():
    logits = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    ids, gates = O.select_topk(logits, 3)
    assert list(ids[0]) == [1, 2, 4]
    np.testing.assert_allclose(gates[0], [1 / 3] * 3, rtol=1e-15)


def test_single_expert_is_dense_geglu_mlp():
    # one expert, no routing freedom: the FFN equals a textbook GeGLU MLP
    lw = _tiny_layer(E=1, seed=4)
    D, F = 256, 128
    lay = O.blob_layout(D, F)
    blob = lw.experts[0]
    sec = lambda n: blob[lay[n][0]:lay[n][0] + lay[n][1]]
    wg = torch.tensor(O._weights_bitwise(sec("gate.codes"), sec("gate.meta"), F, D, 4))
    wu = torch.tensor(O._weights_bitwise(sec("up.codes"), sec("up.meta"), F, D, 4))
    wd = torch.tensor(O._weights_bitwise(sec("down.codes"), sec("down.meta"), D, F, 4))
    x = torch.randn(3, D, dtype=torch.float64, generator=torch.Generator().manual_seed(0))
    ref = torch.nn.functional.linear(
        torch.nn.functional.gelu(torch.nn.functional.linear(x, wg), approximate="tanh")
        * torch.nn.functional.linear(x, wu), wd)
    y = O.expert_forward(x.numpy(), blob, D, F)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-10)


@pytest.mark.parametrize("seed,E,k,T,D,F,Fs", [
    (0, 16, 4, 4, 256, 128, 256),
    (1, 8, 2, 8, 128, 64, 0),
    (2, 16, 16, 3, 64, 64, 128),
    (3, 5, 1, 6, 192, 128, 64),
])
def test_oracle_matches_dense_bruteforce(seed, E, k, T, D, F, Fs):
    cfg = gen.MoEConfig("v", D=D, E=E, F=F, F_shared=Fs, k=k, T=T, x_dtype="fp16")
    lw = gen.layer_weights(seed, 0, cfg)
    x = O.activations_to_float(gen.activations(seed, 0, 0, T, D, "fp16"), "fp16")
    bias = gen.zipf_bias(seed, 0, E, 1.0) if seed % 2 else None
    ref = O.dense_bruteforce(x, lw, k, bias)
    got = O.layer_forward(x, lw, k, bias)
    rel = np.linalg.norm(got["out"] - ref["out"]) / np.linalg.norm(ref["out"])
    assert rel <= 1e-10
    w = np.zeros((T, E))
    for t in range(T):
        w[t, got["ids"][t]] = got["gates"][t]
    np.testing.assert_allclose(w, ref["weights"], atol=1e-12)
    assert np.allclose(got["gates"].sum(axis=1), 1.0, atol=1e-12)
    # fp32 dequantise-and-matmul variant stays within 1e-6 of float64
    g32 = O.layer_forward(x, lw, k, bias, ids=got["ids"], dtype=np.float32)
    rel32 = np.linalg.norm(g32["out"] - got["out"]) / np.linalg.norm(got["out"])
    assert rel32 <= 1e-6


def test_combine_handworked():
    """One token, two routed outputs and a shared one, worked by hand:
    out = ys + 0.25 y0 + 0.75 y1 = [10 + 0.25 + 3, 20 + 0.5 + 3.75, 30 + 0.75 + 4.5]."""
    y = np.array([[[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]]])
    g = np.array([[0.25, 0.75]])
    ys = np.array([[10.0, 20.0, 30.0]])
    assert O.combine(y, g, ys).tolist() == [[13.25, 24.25, 35.25]]
    # without a shared expert the routed part alone
    assert O.combine(y, g, None).tolist() == [[3.25, 4.25, 5.25]]
    # a one-hot gate picks that output
    assert O.combine(y, np.array([[0.0, 1.0]]), None).tolist() == [[4.0, 5.0, 6.0]]


@pytest.mark.parametrize("seed,E,k", [(0, 16, 4), (3, 8, 8)])
def test_combine_equals_dense_bruteforce(seed, E, k):
    """combine of the oracle's per-slot outputs, gates and shared output is
    the dense evaluation of every expert weighted by the masked,
    renormalised softmax (an independent decoder and evaluation)."""
    lw = _tiny_layer(seed, E=E)
    x = O.activations_to_float(gen.activations(seed, 0, 0, 3, 256, "fp16"), "fp16")
    r = O.layer_forward(x, lw, k)
    ref = O.dense_bruteforce(x, lw, k)
    out = O.combine(r["y"], r["gates"], r["y_shared"])
    assert np.linalg.norm(out - ref["out"]) / np.linalg.norm(ref["out"]) < 1e-10


# ---------------------------------------------------------------- activation decoding
_ACT_EDGES = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x4000,
              0xC000, 0x7F7F, 0xFF7F, 0x3C00, 0x7BFF, 0x0400, 0x03FF, 0x3555]


def test_activations_to_float_literals():
    """Bit patterns decoded by hand from the IEEE layouts."""
    bf = O.activations_to_float(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x4049],
                                         np.uint16), "bf16")
    assert bf[0] == 1.0 and bf[1] == -2.0
    assert bf[2] == 2.0 ** -133                      # smallest bf16 subnormal
    assert bf[3] == (2 - 2.0 ** -7) * 2.0 ** 127     # largest finite bf16
    assert bf[4] == 0.0 and math.copysign(1.0, bf[4]) == -1.0
    assert bf[5] == 3.140625                         # 0x4049: 1.5703125 * 2
    hf = O.activations_to_float(np.array([0x3C00, 0x0001, 0x7BFF, 0xC000, 0x0400, 0x3555],
                                         np.uint16), "fp16")
    assert hf[0] == 1.0 and hf[1] == 2.0 ** -24 and hf[2] == 65504.0 and hf[3] == -2.0
    assert hf[4] == 2.0 ** -14                       # smallest normal fp16
    assert hf[5] == 0.333251953125                   # 0x3555: (1 + 341/1024) / 4


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_activations_to_float_matches_torch(dtype):
    """Every finite bit pattern (all 65,536 minus NaN/inf) against torch's own
    bfloat16 / float16 types widened to float64."""
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    ref = torch.from_numpy(u.view(np.int16)).view(tdt).double().numpy()
    fin = np.isfinite(ref)
    got = O.activations_to_float(u, dtype)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    edges = np.array(_ACT_EDGES, np.uint16)
    assert np.array_equal(O.activations_to_float(edges, dtype),
                          torch.from_numpy(edges.view(np.int16)).view(tdt).double().numpy(),
                          equal_nan=True)


# ---------------------------------------------------------------- blob sections
def test_blob_layout_offsets_handworked():
    """Section offsets worked by hand.  D = 2816, F = 704: codes [704, 2816]
    at 4 bits are 991,232 B, metas 44 x 704 x 4 = 123,904 B and
    11 x 2816 x 4 = 123,904 B, all multiples of 256.  D = 256, F = 128 (the
    tiny config): codes 16,384 B, metas 2,048 B."""
    lay = O.blob_layout(2816, 704)
    assert [lay[n][0] for n in ("gate.codes", "up.codes", "down.codes", "gate.meta", "up.meta",
                                "down.meta")] == [0, 991_232, 1_982_464, 2_973_696, 3_097_600,
                                                  3_221_504]
    assert lay["total"][1] == 3_345_408
    tiny = O.blob_layout(256, 128)
    assert [tiny[n] for n in ("gate.codes", "up.codes", "down.codes", "gate.meta", "up.meta",
                              "down.meta")] == [(0, 16384), (16384, 16384), (32768, 16384),
                                                (49152, 2048), (51200, 2048), (53248, 2048)]
    assert tiny["total"][1] == 55_296
    # a width whose sections need padding: D = 64, F = 64 -> 2,048 B codes,
    # 256 B metas: no padding either; D = 64, F = 192 -> meta 192 x 4 = 768 B
    odd = O.blob_layout(64, 192)
    assert odd["gate.meta"] == (18432, 768) and odd["up.meta"] == (19200, 768)
    assert odd["down.meta"] == (19968, 3 * 64 * 4) and odd["total"][1] == 20736


def test_blob_layout_matches_generator_and_header():
    """The oracle's sections equal the generator's and follow the order the
    C header documents."""
    for D, F in [(2816, 704), (2816, 2112), (256, 128), (64, 192)]:
        assert O.blob_layout(D, F) == gen.blob_sections(D, F)
    hdr = open(os.path.join(os.path.dirname(GOLDEN), "..", "include", "moe.h")).read()
    i = hdr.index("Expert blob")
    order = []
    for name in ("gate.codes", "up.codes", "down.codes", "gate.meta", "up.meta", "down.meta"):
        order.append(hdr.index(name, i))
    assert order == sorted(order)
    lay = O.blob_layout(2816, 704)
    offs = [lay[n][0] for n in ("gate.codes", "up.codes", "down.codes", "gate.meta", "up.meta",
                                "down.meta")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)


# ---------------------------------------------------------------- block norms and residual
def test_rms_norm_handworked_and_torch():
    """x = [3, 4]: mean square 12.5, rms 3.5355...; with w = 0 and eps = 0 the
    output is [3, 4] / 3.5355 = [0.8485, 1.1314]; and random rows against
    torch.nn.functional.rms_norm with weight (1 + w)."""
    got = O.rms_norm(np.array([[3.0, 4.0]]), np.zeros(2), eps=0.0)
    np.testing.assert_allclose(got, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)
    assert abs(got[0, 0] - 0.848528137423857) < 1e-12
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 2816)) * 3
    w = rng.standard_normal(2816) * 0.1
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (2816,),
                                       weight=torch.from_numpy(1.0 + w), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), ref, rtol=1e-12, atol=1e-14)
    # w = 0: every row has unit root mean square (up to eps)
    u = O.rms_norm(x, np.zeros(2816), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(u * u, axis=1)), 1.0, rtol=1e-12)


def test_round_to_bf16_ties_and_torch():
    """1 + 2^-8 is halfway between bf16 1 and 1 + 2^-7: ties to even gives 1;
    1 + 3 * 2^-8 rounds up to 1 + 2^-6.  Random values against torch."""
    assert O.round_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert O.round_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82
    v = np.random.default_rng(3).standard_normal(10000) * 10
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(O.round_to_bf16(v), ref.view(np.uint16))


def test_block_forward_structure():
    """out - x has the root mean square of (1 + w_post) per row, and the
    block's layer input is the rounded pre-norm of x."""
    lw = _tiny_layer(0)
    x = O.activations_to_float(gen.activations(5, 0, 0, 3, 256, "fp16"), "fp16") * 4
    rng = np.random.default_rng(8)
    w_pre, w_post = rng.standard_normal(256) * 0.1, np.zeros(256)
    r = O.block_forward(x, lw, 4, w_pre, w_post, eps=0.0)
    d = r["out"] - x
    np.testing.assert_allclose(np.sqrt(np.mean(d * d, axis=1)), 1.0, rtol=1e-12)
    u = O.activations_to_float(O.round_to_bf16(O.rms_norm(x, w_pre, 0.0)), "bf16")
    assert np.array_equal(r["u"], u)
    np.testing.assert_allclose(r["moe"], O.layer_forward(u, lw, 4)["out"], rtol=1e-13)


# ---------------------------------------------------------------- permutation
def test_permutation_handworked():
    ids = np.array([[2, 0], [0, 1], [2, 1]])
    counts, offsets, perm, inv = O.permutation(ids, 3)
    assert list(counts) == [2, 2, 2]
    assert list(offsets) == [0, 2, 4, 6]
    # flat pairs: 0:(t0,e2) 1:(t0,e0) 2:(t1,e0) 3:(t1,e1) 4:(t2,e2) 5:(t2,e1)
    assert list(perm) == [1, 2, 3, 5, 0, 4]
    assert list(inv) == [4, 0, 1, 2, 5, 3]


def test_permutation_invariants_random():
    rng = np.random.default_rng(7)
    E, T, k = 128, 128, 8
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, perm, inv = O.permutation(ids, E)
    flat = ids.reshape(-1)
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(inv[perm], np.arange(T * k))
    assert np.array_equal(perm[inv], np.arange(T * k))
    assert np.array_equal(np.bincount(flat, minlength=E), counts)


# ---------------------------------------------------------------- LFU pool model
def _golden_lfu():
    with open(os.path.join(GOLDEN, "lfu_trace.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    slots, E = map(int, lines[0].split())
    steps = []
    for l in lines[1:]:
        _, rest = l.split(":", 1)
        ids_s, ev_s = rest.split(";")
        ids = [int(v) for v in ids_s.split()]
        evs = []
        for item in ev_s.split():
            e, s, h, v = item.split(":")
            evs.append((int(e), int(s), h == "hit", int(v)))
        steps.append((ids, evs))
    return slots, E, steps


def test_lfu_handworked_trace():
    slots, E, steps = _golden_lfu()
    c = O.LFUCache(slots, E)
    for ids, evs in steps:
        assert c.access(ids) == evs


def test_lru_handworked_trace():
    """Two slots, one expert per token: 0, 0, 1, 2, 0.  At the fourth token
    LRU evicts expert 0 (last used at token 1; expert 1 at token 2), where
    LFU would evict expert 1 (used once against twice); at the fifth, expert
    0 misses and expert 1 (token 2, older than expert 2 at token 3) goes."""
    c = O.LRUCache(2, 4)
    got = [c.access([e]) for e in (0, 0, 1, 2, 0)]
    assert got == [[(0, 0, False, -1)], [(0, 0, True, -1)], [(1, 1, False, -1)],
                   [(2, 0, False, 0)], [(0, 1, False, 1)]]
    f = O.LFUCache(2, 4)
    lfu = [f.access([e]) for e in (0, 0, 1, 2)]
    assert lfu[3] == [(2, 1, False, 1)]  # the policies part here


def test_lfu_never_evicts_needed_and_bounds():
    rng = np.random.default_rng(11)
    c = O.LFUCache(16, 128)
    for _ in range(300):
        ids = rng.choice(128, size=8, replace=False)
        evs = c.access(ids)
        assert all(v not in ids for (_, _, _, v) in evs)
        assert sum(1 for s in c.expert_in if s >= 0) <= 16
        assert all(c.slot_of[e] >= 0 for e in ids)


# ---------------------------------------------------------------- sizes the pages print
def test_storage_sizes_match_pages():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    blob = O.blob_layout(2816, 704)["total"][1]
    assert blob == 3_345_408
    assert abs(blob / 1e6 - fig["expert_bytes_MB"]["value"]) / fig["expert_bytes_MB"]["value"] < 0.01
    total = blob * fig["experts_per_layer"]["value"] * fig["layers"]["value"]
    assert abs(total / 1e9 - fig["experts_total_GB"]["value"]) / fig["experts_total_GB"]["value"] < 0.01
    lo_hit, hi_hit = fig["cache_hit_rate"]["value"]
    per_token = fig["top_k"]["value"] * fig["layers"]["value"] * blob
    miss_lo, miss_hi = per_token * (1 - hi_hit) / 1e6, per_token * (1 - lo_hit) / 1e6
    pages_lo, pages_hi = fig["ssd_bytes_per_token_MB"]["value"]
    assert miss_lo < pages_hi and miss_hi > pages_lo  # ranges overlap
    assert abs(miss_lo - pages_lo) / pages_lo < 0.05 and abs(miss_hi - pages_hi) / pages_hi < 0.05
    # the generator's layout arithmetic agrees with the oracle's
    assert gen.blob_bytes(2816, 704) == blob
    assert gen.blob_bytes(2816, 2112) == O.blob_layout(2816, 2112)["total"][1] == 10_036_224


# ---------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible oracle mistakes and check that some pin fails."""
    # (1) scale and bias swapped while unpacking meta -> one-hot pin fails
    orig = O.unpack_meta

    def swapped(meta, rows, cols):
        s, b = orig(meta, rows, cols)
        return b, s
    monkeypatch.setattr(O, "unpack_meta", swapped)
    with pytest.raises(AssertionError):
        test_onehot_selects_one_dequantised_column()
    monkeypatch.setattr(O, "unpack_meta", orig)

    # (2) gate and up exchanged inside the expert -> dense GeGLU pin fails
    orig_w = O.expert_weights

    def exchanged(blob, D, F, dtype=np.float64):
        wg, wu, wd = orig_w(blob, D, F, dtype)
        return wu, wg, wd
    monkeypatch.setattr(O, "expert_weights", exchanged)
    with pytest.raises(AssertionError):
        test_single_expert_is_dense_geglu_mlp()
    monkeypatch.setattr(O, "expert_weights", orig_w)

    # (3) gates as softmax over all experts without renormalising -> brute force pin fails
    orig_sel = O.select_topk

    def unnormalised(logits, k):
        ids, _ = orig_sel(logits, k)
        p = scipy.special.softmax(logits, axis=1)
        return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)
    monkeypatch.setattr(O, "select_topk", unnormalised)
    with pytest.raises(AssertionError):
        test_oracle_matches_dense_bruteforce(0, 16, 4, 4, 256, 128, 256)
    monkeypatch.setattr(O, "select_topk", orig_sel)

    # (4) erf-form GELU -> golden points fail
    monkeypatch.setattr(O, "gelu_tanh", lambda x: 0.5 * np.asarray(x) * (1 + scipy.special.erf(np.asarray(x) / math.sqrt(2))))
    with pytest.raises(AssertionError):
        test_gelu_tanh_golden_points()

    # (5) combine that drops the shared output -> hand-worked combine fails
    orig_c = O.combine
    monkeypatch.setattr(O, "combine", lambda y, g, ys: orig_c(y, g, None))
    with pytest.raises(AssertionError):
        test_combine_handworked()
    monkeypatch.setattr(O, "combine", orig_c)

    # (6) bf16 widened by a shift of 8 instead of 16 -> literal decoding fails
    orig_a = O.activations_to_float

    def shifted(x_bits, x_dtype):
        if x_dtype == "bf16":
            u = np.asarray(x_bits, dtype=np.uint16)
            return (u.astype(np.uint32) << 8).view(np.float32).astype(np.float64)
        return orig_a(x_bits, x_dtype)
    monkeypatch.setattr(O, "activations_to_float", shifted)
    with pytest.raises(AssertionError):
        test_activations_to_float_literals()
    monkeypatch.setattr(O, "activations_to_float", orig_a)

    # (7) blob sections with gate and up codes exchanged -> offsets fail
    orig_b = O.blob_layout

    def exchanged_sections(D, F):
        lay = dict(orig_b(D, F))
        lay["gate.codes"], lay["up.codes"] = lay["up.codes"], lay["gate.codes"]
        return lay
    monkeypatch.setattr(O, "blob_layout", exchanged_sections)
    with pytest.raises(AssertionError):
        test_blob_layout_offsets_handworked()
    monkeypatch.setattr(O, "blob_layout", orig_b)

    # (8) RMSNorm without the (1 + w) offset -> the torch comparison fails
    orig_n = O.rms_norm

    def no_offset(v, w, eps=O.NORM_EPS):
        return orig_n(v, np.asarray(w) - 1.0, eps)
    monkeypatch.setattr(O, "rms_norm", no_offset)
    with pytest.raises(AssertionError):
        test_rms_norm_handworked_and_torch()
    monkeypatch.setattr(O, "rms_norm", orig_n)
