"""Seeded synthetic inputs for the routed int4 MoE FFN layer.

Test and benchmark infrastructure shared by the CPU oracle and the HIP path.
It holds none of the layer's arithmetic: it draws random codes, scales,
biases and activations, and places them in the storage layout the kernels
read (the pages stress that the experts live on disk in exactly the packed
4-bit layout the GPU kernel consumes -- stork.ai blog, "El arma secreta de
Apple: memoria unificada").  Nothing here dequantises, multiplies, routes or
sorts.

Storage layout of one affine-quantised matrix W[R, C] (R output rows, C input
columns, ``bits`` in {4, 8}, one fp16 scale and one fp16 bias per 64
consecutive columns of a row; MLX-style affine format named on
es.news.hada.io, "Estructura de ejecucion para reducir memoria", and
imasters.com.br, "O truque"):

* codes: 16-byte chunks.  A chunk holds ``n = 128 / bits`` consecutive
  columns of one row; chunk (r, cc) with ``cc = c // n`` sits at byte offset
  ``(cc * R + r) * 16`` (chunk-major: one chunk position for every row, then
  the next).  Inside the chunk the code of column c occupies bits
  ``[bits * (c % n), bits * (c % n) + bits)`` of the little-endian 128-bit
  value.
* meta: one little-endian u32 per (group, row) at index ``(c // 64) * R + r``;
  bits 0-15 hold the fp16 scale, bits 16-31 the fp16 bias.

Expert blob (one GLU expert of model width D and hidden width F, 4-bit):
sections gate.codes [F, D], up.codes [F, D], down.codes [D, F], gate.meta,
up.meta, down.meta, in that order, each starting on a 256-byte boundary.
At D = 2816, F = 704 a blob is 3,345,408 bytes (the pages quote 3.36 MB per
expert: hndistilled.com, "Enfoque tecnico"; es.news.hada.io, HN thread).
"""
from __future__ import annotations

import dataclasses
import os
import math
from typing import Dict, Tuple

import numpy as np

GROUP = 64
ALIGN = 256

# spawn-key kinds: every tensor has its own child seed so that any single
# expert, router or activation block can be regenerated on its own.
KIND_EXPERT, KIND_SHARED, KIND_ROUTER, KIND_X, KIND_ZIPF, KIND_NORM = 0, 1, 2, 3, 4, 5
PART_GATE, PART_UP, PART_DOWN = 0, 1, 2


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    D: int            # model width
    E: int            # routed experts per layer
    F: int            # routed expert hidden width
    F_shared: int     # shared expert hidden width (0: no shared expert)
    k: int            # experts selected per token
    T: int            # tokens per call
    x_dtype: str      # "fp16" or "bf16"
    layers: int = 1   # distinct seeded layers (replicas or a stack)
    tokens: int = 1   # tokens per layer sequence (stack / streamed configs)
    chunks: int = 1   # prefill chunks
    beta: float = 0.0  # Zipf skew of the router-logit bias (0: no bias)
    slots: int = 0    # HBM expert slots per layer (streamed config)


# Zipf skew parameters found by oracle/calibrate_zipf.py (seed 0):
#   stack / streamed decode: mean repeat-from-previous-token in [0.60, 0.70];
#   prefill: largest per-expert row count of a 128-token chunk in [50, 60].
BETA_STACK = 6.5
BETA_PREFILL = 1.5

CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", D=256, E=16, F=128, F_shared=256, k=4, T=4,
                      x_dtype="fp16"),
    "decode": MoEConfig("decode", D=2816, E=128, F=704, F_shared=2112, k=8,
                        T=1, x_dtype="bf16", layers=16),
    "stack30": MoEConfig("stack30", D=2816, E=128, F=704, F_shared=2112, k=8,
                         T=1, x_dtype="bf16", layers=30, tokens=256,
                         beta=BETA_STACK),
    "prefill": MoEConfig("prefill", D=2816, E=128, F=704, F_shared=2112, k=8,
                         T=128, x_dtype="bf16", layers=2, chunks=8,
                         beta=BETA_PREFILL),
    "streamed": MoEConfig("streamed", D=2816, E=128, F=704, F_shared=2112,
                          k=8, T=1, x_dtype="bf16", layers=30, tokens=256,
                          beta=BETA_STACK, slots=16),
}


# --------------------------------------------------------------------------
# layout arithmetic (sizes and offsets only)
# --------------------------------------------------------------------------
def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def codes_bytes(rows: int, cols: int, bits: int) -> int:
    return rows * cols * bits // 8


def meta_bytes(rows: int, cols: int) -> int:
    return (cols // GROUP) * rows * 4


def blob_sections(D: int, F: int) -> Dict[str, Tuple[int, int]]:
    """(offset, nbytes) of every section of a 4-bit GLU expert blob."""
    sizes = [
        ("gate.codes", codes_bytes(F, D, 4)),
        ("up.codes", codes_bytes(F, D, 4)),
        ("down.codes", codes_bytes(D, F, 4)),
        ("gate.meta", meta_bytes(F, D)),
        ("up.meta", meta_bytes(F, D)),
        ("down.meta", meta_bytes(D, F)),
    ]
    out, off = {}, 0
    for name, n in sizes:
        out[name] = (off, n)
        off = _align(off + n)
    out["total"] = (0, off)
    return out


def blob_bytes(D: int, F: int) -> int:
    return blob_sections(D, F)["total"][1]


# --------------------------------------------------------------------------
# packing (structured test inputs)
# --------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Place integer codes [R, C] into the chunk-major byte layout."""
    codes = np.asarray(codes)
    R, C = codes.shape
    if bits not in (4, 8) or C % GROUP:
        raise ValueError("bits must be 4 or 8 and C a multiple of 64")
    if codes.min() < 0 or codes.max() >= (1 << bits):
        raise ValueError("code out of range")
    n = 128 // bits
    # [R, C/n, n] -> [C/n, R, n]
    ch = codes.astype(np.uint8).reshape(R, C // n, n).transpose(1, 0, 2)
    if bits == 8:
        return np.ascontiguousarray(ch).reshape(-1)
    lo = ch[:, :, 0::2]
    hi = ch[:, :, 1::2]
    return np.ascontiguousarray(lo | (hi << 4)).reshape(-1)


def pack_meta(scale_f16: np.ndarray, bias_f16: np.ndarray) -> np.ndarray:
    """[R, C/64] fp16 scale and bias -> u32 meta words, group-major."""
    s = np.asarray(scale_f16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    b = np.asarray(bias_f16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return np.ascontiguousarray((s | (b << 16)).T).reshape(-1)


def assemble_blob(D: int, F: int, parts: Dict[str, np.ndarray]) -> np.ndarray:
    """Write packed sections (bytes / u32 arrays) into one blob."""
    sec = blob_sections(D, F)
    blob = np.zeros(sec["total"][1], dtype=np.uint8)
    for name, arr in parts.items():
        off, n = sec[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        if raw.size != n:
            raise ValueError(f"{name}: {raw.size} bytes, expected {n}")
        blob[off:off + n] = raw
    return blob


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------
def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    words = rng.bit_generator.random_raw((n + 7) // 8).astype(np.uint64)
    return words.view(np.uint8)[:n]


def _affine_meta(rng, rows, cols, smin, smax, bmax):
    g = cols // GROUP
    scale = rng.uniform(smin, smax, size=(rows, g)).astype(np.float16)
    bias = rng.uniform(-bmax, bmax, size=(rows, g)).astype(np.float16)
    return scale, bias


def random_matrix(rng, rows, cols, bits, smin, smax, bmax):
    """Uniform codes plus U(smin, smax) scales and U(-bmax, bmax) biases."""
    codes = _random_bytes(rng, codes_bytes(rows, cols, bits))
    scale, bias = _affine_meta(rng, rows, cols, smin, smax, bmax)
    return codes, pack_meta(scale, bias)


def expert_blob(seed: int, layer: int, expert: int, D: int, F: int,
                shared: bool = False, out: np.ndarray | None = None) -> np.ndarray:
    """One 4-bit GLU expert: q~U{0..15}, scale~U(0.005,0.02), bias~U(-0.1,0.1)."""
    kind = KIND_SHARED if shared else KIND_EXPERT
    parts = {}
    for part, name, (R, C) in ((PART_GATE, "gate", (F, D)), (PART_UP, "up", (F, D)),
                               (PART_DOWN, "down", (D, F))):
        rng = _rng(seed, kind, layer, expert, part)
        codes, meta = random_matrix(rng, R, C, 4, 0.005, 0.02, 0.1)
        parts[name + ".codes"] = codes
        parts[name + ".meta"] = meta
    blob = assemble_blob(D, F, parts)
    if out is not None:
        out[...] = blob
        return out
    return blob


@dataclasses.dataclass
class RouterQ:
    codes: np.ndarray   # uint8 bytes, chunk-major, 8-bit codes
    meta: np.ndarray    # uint32 words
    rows: int
    cols: int
    bits: int = 8


def router(seed: int, layer: int, E: int, D: int) -> RouterQ:
    """8-bit router: q~U{0..255}, scale~U(0.005,0.02)/17, bias~U(-0.1,0.1)."""
    rng = _rng(seed, KIND_ROUTER, layer)
    codes, meta = random_matrix(rng, E, D, 8, 0.005 / 17, 0.02 / 17, 0.1)
    return RouterQ(codes, meta, E, D, 8)


def _round_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activations(seed: int, layer: int, stream: int, T: int, D: int,
                dtype: str) -> np.ndarray:
    """x ~ N(0, 1) rounded to fp16 or bf16; returned as uint16 bit patterns."""
    rng = _rng(seed, KIND_X, layer, stream)
    x = rng.standard_normal((T, D)).astype(np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _round_bf16_bits(x)
    raise ValueError(dtype)


def norm_weights(seed: int, layer: int, D: int) -> Tuple[np.ndarray, np.ndarray]:
    """The residual block's two RMSNorm weight vectors (pre, post), fp32,
    w ~ N(0, 0.25^2): effective scales 1 + w scattered around 1."""
    rng = _rng(seed, KIND_NORM, layer)
    w = (0.25 * rng.standard_normal((2, D))).astype(np.float32)
    return w[0].copy(), w[1].copy()


def residual_stream(seed: int, layer: int, stream: int, T: int, D: int,
                    dtype: str) -> np.ndarray:
    """The residual stream entering a block: N(0, 1) rows with a per-row scale
    drawn log-uniformly in [1/4, 16] (the stream's norm grows along the layer
    stack), rounded to fp16 or bf16; uint16 bit patterns."""
    rng = _rng(seed, KIND_X, layer, stream, 1)
    scale = np.exp(rng.uniform(np.log(0.25), np.log(16.0), size=(T, 1)))
    x = (rng.standard_normal((T, D)) * scale).astype(np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _round_bf16_bits(x)
    raise ValueError(dtype)


def zipf_bias(seed: int, layer: int, E: int, beta: float, s: float = 1.1) -> np.ndarray:
    """Per-layer logit bias -beta * s * ln(rank): log of a Zipf(s) pmf up to a
    constant, over a seeded random ranking of the experts."""
    if beta == 0.0:
        return np.zeros(E, dtype=np.float32)
    rng = _rng(seed, KIND_ZIPF, layer)
    order = rng.permutation(E)
    rank = np.empty(E, dtype=np.float64)
    rank[order] = np.arange(1, E + 1)
    return (-beta * s * np.log(rank)).astype(np.float32)


# --------------------------------------------------------------------------
# whole layers
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LayerWeights:
    router: RouterQ
    experts: np.ndarray        # uint8 [E, blob_bytes(D, F)]
    shared: np.ndarray | None  # uint8 [blob_bytes(D, F_shared)]
    D: int
    F: int
    F_shared: int


def layer_weights(seed: int, layer: int, cfg: MoEConfig,
                  experts_out: np.ndarray | None = None) -> LayerWeights:
    nb = blob_bytes(cfg.D, cfg.F)
    experts = experts_out if experts_out is not None else np.empty((cfg.E, nb), np.uint8)
    for e in range(cfg.E):
        expert_blob(seed, layer, e, cfg.D, cfg.F, out=experts[e])
    shared = (expert_blob(seed, layer, 0, cfg.D, cfg.F_shared, shared=True)
              if cfg.F_shared else None)
    return LayerWeights(router(seed, layer, cfg.E, cfg.D), experts, shared,
                        cfg.D, cfg.F, cfg.F_shared)


def bytes_to_f16(u16: np.ndarray) -> np.ndarray:
    return np.asarray(u16, dtype=np.uint16).view(np.float16)


def algorithmic_decode_bytes(cfg: MoEConfig) -> int:
    """Bytes one decode token reads in one layer: router, k expert blobs,
    the shared expert and the activation vector in and out."""
    r = codes_bytes(cfg.E, cfg.D, 8) + meta_bytes(cfg.E, cfg.D)
    e = cfg.k * blob_bytes(cfg.D, cfg.F)
    s = blob_bytes(cfg.D, cfg.F_shared) if cfg.F_shared else 0
    act = cfg.D * 2 + cfg.D * 4
    return r + e + s + act


def store_stride(D: int, F: int) -> int:
    """Bytes per blob in an expert file: the blob rounded up to 4096."""
    return (blob_bytes(D, F) + 4095) // 4096 * 4096


def write_expert_file(path: str, seed: int, n_layers: int, cfg: MoEConfig) -> int:
    """Every routed expert blob of layers 0..n_layers-1 into one file, blob
    (l, e) at (l * E + e) * store_stride, zero padded; returns the file size.
    The same seeded bytes as layer_weights()."""
    stride = store_stride(cfg.D, cfg.F)
    nb = blob_bytes(cfg.D, cfg.F)
    buf = np.zeros((cfg.E, stride), dtype=np.uint8)
    with open(path, "wb") as f:
        for l in range(n_layers):
            for e in range(cfg.E):
                expert_blob(seed, l, e, cfg.D, cfg.F, out=buf[e, :nb])
            f.write(buf.tobytes())
        f.flush()
        os.fsync(f.fileno())
    return n_layers * cfg.E * stride
