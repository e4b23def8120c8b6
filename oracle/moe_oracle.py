"""Plain CPU oracle for the routed int4 Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never imports it; it reads the packed arrays the
seeded generator writes and unpacks them itself.

What the layer computes (the pages' per-layer token loop: es.news.hada.io,
"Proceso de generacion de tokens"; yodev.dev, "Por que funciona: el A4B del
nombre"; imasters.com.br, "O truque"; stork.ai blog, "Por que la mayor parte
de tu modelo de IA es peso muerto"):

1. an 8-bit affine router scores every expert from the layer input;
2. the 8 highest-scoring of 128 experts are selected and given gate weights;
3. each selected expert is a 4-bit affine GLU feed-forward block;
4. a resident shared expert runs on every token and its output is added to
   the gate-weighted sum of the routed outputs.

Readings where the pages are silent (each is listed with its reason in the
design notes):

* affine format (MLX affine, group 64): ``w = scale * q + bias`` with
  unsigned codes ``q`` in ``[0, 2**bits)`` and one fp16 scale and bias per 64
  consecutive input columns of a row;
* router logits are ``x @ Wr.T`` plus an optional per-expert logit bias (used
  for Zipf-skewed routing), with no other scaling;
* selection keeps the k largest logits, larger first, equal logits going to
  the lower expert index; the decision is taken on logits rounded to fp32,
  the precision the GPU path scores in;
* gate weights are the softmax over the k selected logits;
* the GLU activation is GELU in its tanh form, ``h = gelu(x Wg^T) * (x Wu^T)``;
* the shared expert takes the same x and is added with weight 1.

Arithmetic is float64 by default (dequantised weights are exact in float64);
``dtype=np.float32`` gives the fp32 dequantise-and-matmul variant.

The block around the layer (a reading: the pages define no norm): a
Gemma-style pre-norm RMSNorm of the residual stream, rounded to bf16, feeds
the layer, and out = x + RMSNorm(layer output) with its own weights.

Parity pins (tests/test_oracle_pins.py): hand-built code words, one-hot and
constant-code closed forms, GELU values at fixed points, x = 0, k = E softmax,
a single-expert dense GeGLU MLP, an independently decoded brute-force dense
evaluation of all experts, permutation invariants, a hand-worked LFU trace,
and the pages' storage sizes.  "Parity unpinned": fidelity to the real
checkpoint's router scaling, activation variant and block norms -- the pages
state none of them.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

GROUP = 64
ALIGN = 256


# --------------------------------------------------------------------------
# storage format
# --------------------------------------------------------------------------
def unpack_codes(codes: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """Integer codes [rows, cols] from the chunk-major packed bytes.

    A 16-byte chunk holds 128/bits consecutive columns of one row; chunk
    (r, cc) is stored at byte (cc * rows + r) * 16; a column's code sits at
    bits [bits*j, bits*j + bits) of the little-endian chunk, j its position
    inside the chunk.
    """
    raw = np.asarray(codes).view(np.uint8).reshape(-1)
    n = 128 // bits
    if raw.size != rows * cols * bits // 8:
        raise ValueError("packed size does not match the shape")
    ch = raw.reshape(cols // n, rows, 16)
    if bits == 8:
        vals = ch
    elif bits == 4:
        vals = np.empty((cols // n, rows, 32), dtype=np.uint8)
        vals[:, :, 0::2] = ch & 0x0F
        vals[:, :, 1::2] = ch >> 4
    else:
        raise ValueError("bits must be 4 or 8")
    return vals.transpose(1, 0, 2).reshape(rows, cols).astype(np.int64)


def unpack_meta(meta: np.ndarray, rows: int, cols: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 scale and bias [rows, cols/64] from the group-major u32 words."""
    w = np.asarray(meta).view(np.uint32).reshape(cols // GROUP, rows).T
    scale = (w & 0xFFFF).astype(np.uint16).view(np.float16)
    bias = (w >> 16).astype(np.uint16).view(np.float16)
    return scale, bias


def dequantize(codes, meta, rows, cols, bits, dtype=np.float64) -> np.ndarray:
    """W[r, c] = scale[r, c // 64] * q[r, c] + bias[r, c // 64]."""
    q = unpack_codes(codes, rows, cols, bits).astype(dtype)
    scale, bias = unpack_meta(meta, rows, cols)
    s = np.repeat(scale.astype(dtype), GROUP, axis=1)
    b = np.repeat(bias.astype(dtype), GROUP, axis=1)
    prod = (s * q).astype(dtype)
    return (prod + b).astype(dtype)


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def blob_layout(D: int, F: int) -> Dict[str, Tuple[int, int]]:
    """Sections of a 4-bit GLU expert blob: gate, up, down codes then metas."""
    cb = lambda r, c: r * c // 2
    mb = lambda r, c: (c // GROUP) * r * 4
    order = [("gate.codes", cb(F, D)), ("up.codes", cb(F, D)), ("down.codes", cb(D, F)),
             ("gate.meta", mb(F, D)), ("up.meta", mb(F, D)), ("down.meta", mb(D, F))]
    out, off = {}, 0
    for name, n in order:
        out[name] = (off, n)
        off = _align(off + n)
    out["total"] = (0, off)
    return out


def expert_weights(blob: np.ndarray, D: int, F: int, dtype=np.float64):
    """Dequantised (Wg [F, D], Wu [F, D], Wd [D, F]) of one expert blob."""
    lay = blob_layout(D, F)
    raw = np.asarray(blob).view(np.uint8).reshape(-1)
    if raw.size < lay["total"][1]:
        raise ValueError("blob too small")

    def sec(name):
        off, n = lay[name]
        return raw[off:off + n]

    wg = dequantize(sec("gate.codes"), sec("gate.meta").view(np.uint32), F, D, 4, dtype)
    wu = dequantize(sec("up.codes"), sec("up.meta").view(np.uint32), F, D, 4, dtype)
    wd = dequantize(sec("down.codes"), sec("down.meta").view(np.uint32), D, F, 4, dtype)
    return wg, wu, wd


def activations_to_float(x_bits: np.ndarray, x_dtype: str) -> np.ndarray:
    """fp16 / bf16 bit patterns -> exact float64 values."""
    u = np.asarray(x_bits, dtype=np.uint16)
    if x_dtype == "fp16":
        return u.view(np.float16).astype(np.float64)
    if x_dtype == "bf16":
        with np.errstate(invalid="ignore"):  # signalling NaN patterns stay NaN
            return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(x_dtype)


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------
def gelu_tanh(x):
    """GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x)
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x * x * x)))


def router_logits(x: np.ndarray, router, logit_bias=None, dtype=np.float64) -> np.ndarray:
    """logits[t, e] = sum_d x[t, d] * Wr[e, d] (+ logit_bias[e])."""
    wr = dequantize(router.codes, router.meta, router.rows, router.cols, router.bits, dtype)
    l = np.asarray(x, dtype=dtype) @ wr.T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=dtype)[None, :]
    return l


def select_topk(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token and their softmax gate weights.

    Order: descending logit as rounded to fp32, ties to the lower index.
    Gates: softmax over the k selected logits (at full precision).
    """
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    l32 = logits.astype(np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(l32[t, e]), e))[:k]
        ids[t] = order
        sel = logits[t, order].astype(np.float64)
        z = np.exp(sel - sel.max())
        gates[t] = z / z.sum()
    return ids, gates


def expert_forward(x_rows: np.ndarray, blob: np.ndarray, D: int, F: int,
                   dtype=np.float64, weights=None) -> np.ndarray:
    """GLU expert: y = (gelu(x Wg^T) * (x Wu^T)) Wd^T."""
    wg, wu, wd = weights if weights is not None else expert_weights(blob, D, F, dtype)
    x = np.asarray(x_rows, dtype=dtype)
    g = x @ wg.T
    u = x @ wu.T
    h = (gelu_tanh(g) * u).astype(dtype)
    return (h @ wd.T).astype(dtype)


def layer_forward(x: np.ndarray, layer, k: int, logit_bias=None,
                  ids: Optional[np.ndarray] = None, dtype=np.float64) -> Dict[str, np.ndarray]:
    """One MoE layer on tokens x [T, D] (float values).

    ``layer`` carries ``router``, ``experts`` [E, blob], ``shared`` blob or
    None, ``D``, ``F``, ``F_shared``.  If ``ids`` is given, those experts are
    used instead of the router's choice (gates still come from the logits).
    Returns out [T, D], ids, gates, logits, y [T, k, D], y_shared [T, D].
    """
    x = np.asarray(x, dtype=dtype)
    T, D = x.shape
    logits = router_logits(x, layer.router, logit_bias, dtype)
    if ids is None:
        ids, gates = select_topk(logits, k)
    else:
        ids = np.asarray(ids, dtype=np.int32)
        gates = np.empty(ids.shape, dtype=np.float64)
        for t in range(T):
            sel = logits[t, ids[t]].astype(np.float64)
            z = np.exp(sel - sel.max())
            gates[t] = z / z.sum()
    y = np.zeros((T, k, D), dtype=dtype)
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = expert_weights(layer.experts[e], D, layer.F, dtype)
            y[t, j] = expert_forward(x[t:t + 1], None, D, layer.F, dtype, cache[e])[0]
    if layer.shared is not None:
        ys = expert_forward(x, layer.shared, D, layer.F_shared, dtype)
    else:
        ys = np.zeros((T, D), dtype=dtype)
    out = ys.copy()
    for j in range(k):
        out = out + gates[:, j:j + 1].astype(dtype) * y[:, j, :]
    return {"out": out, "ids": ids, "gates": gates, "logits": logits, "y": y, "y_shared": ys}


def combine(y: np.ndarray, gates: np.ndarray, y_shared: Optional[np.ndarray]) -> np.ndarray:
    """out[t] = y_shared[t] + sum_j gates[t, j] * y[t, j], in j order."""
    T, k, D = y.shape
    out = np.zeros((T, D)) if y_shared is None else np.asarray(y_shared, dtype=np.float64).copy()
    for j in range(k):
        out = out + np.asarray(gates[:, j:j + 1], np.float64) * np.asarray(y[:, j, :], np.float64)
    return out


# --------------------------------------------------------------------------
# the transformer block around the layer (synthetic: the pages name the
# normalisation and residual work of a block but do not define it)
# --------------------------------------------------------------------------
NORM_EPS = 1e-6


def rms_norm(v: np.ndarray, w: np.ndarray, eps: float = NORM_EPS) -> np.ndarray:
    """Gemma-style RMSNorm of each row: v / sqrt(mean(v^2) + eps) * (1 + w)."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * (1.0 + np.asarray(w, dtype=np.float64))


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Float values rounded to fp32, then to the nearest bf16 (ties to even),
    as uint16 bits: the rounding decision taken in fp32, as the kernels take
    it."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def block_forward(x: np.ndarray, layer, k: int, w_pre: np.ndarray, w_post: np.ndarray,
                  eps: float = NORM_EPS, logit_bias=None, ids=None,
                  u: Optional[np.ndarray] = None, x_dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """A pre/post-normed residual block around the MoE layer:
    out = x + rms_norm(MoE(u), w_post) with u = rms_norm(x, w_pre) rounded to
    the layer's 16-bit activations (x_dtype, round to nearest even).  ``u``
    (float values) replaces the rounded pre-norm when given: the rounding is
    a decision the GPU takes in its own fp32 arithmetic, and the layer is then
    compared on the same inputs."""
    x = np.asarray(x, dtype=np.float64)
    if u is None:
        v = rms_norm(x, w_pre, eps)
        if x_dtype == "bf16":
            u = activations_to_float(round_to_bf16(v), "bf16")
        elif x_dtype == "fp16":
            u = v.astype(np.float16).astype(np.float64)
        else:
            raise ValueError(x_dtype)
    r = layer_forward(u, layer, k, logit_bias, ids=ids)
    out = x + rms_norm(r["out"], w_post, eps)
    return {"out": out, "u": u, "moe": r["out"], "ids": r["ids"], "gates": r["gates"],
            "logits": r["logits"]}


# --------------------------------------------------------------------------
# brute force: every expert on every token, masked (independent decode path)
# --------------------------------------------------------------------------
def _decode_bitwise(codes: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """Second decoder of the packed codes: gathers each code bit by bit from
    the little-endian bit stream at the position the layout definition gives."""
    raw = np.asarray(codes).view(np.uint8).reshape(-1)
    bitstream = np.unpackbits(raw, bitorder="little").astype(np.int64)
    n = 128 // bits
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    start = ((c // n) * rows + r) * 128 + bits * (c % n)
    q = np.zeros((rows, cols), dtype=np.int64)
    for b in range(bits):
        q += bitstream[start + b] << b
    return q


def _meta_bitwise(meta: np.ndarray, rows: int, cols: int):
    w = np.asarray(meta).view(np.uint32).reshape(-1)
    scale = np.empty((rows, cols // GROUP))
    bias = np.empty((rows, cols // GROUP))
    for r in range(rows):
        for g in range(cols // GROUP):
            v = int(w[g * rows + r])
            scale[r, g] = float(np.uint16(v & 0xFFFF).view(np.float16))
            bias[r, g] = float(np.uint16(v >> 16).view(np.float16))
    return scale, bias


def _weights_bitwise(codes, meta, rows, cols, bits):
    q = _decode_bitwise(codes, rows, cols, bits)
    s, b = _meta_bitwise(meta, rows, cols)
    W = np.empty((rows, cols))
    for c in range(cols):
        W[:, c] = s[:, c // GROUP] * q[:, c] + b[:, c // GROUP]
    return W


def dense_bruteforce(x: np.ndarray, layer, k: int, logit_bias=None) -> Dict[str, np.ndarray]:
    """Evaluate all E experts densely in float64 and weight them with the
    renormalised softmax of all logits masked to the top k (tiny inputs only)."""
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    E = layer.experts.shape[0]
    rt = layer.router
    wr = _weights_bitwise(rt.codes, rt.meta, rt.rows, rt.cols, rt.bits)
    logits = np.einsum("td,ed->te", x, wr)
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, np.float64)[None, :]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    l32 = logits.astype(np.float32)
    mask = np.zeros((T, E))
    for t in range(T):
        # rank of every expert: count of experts that beat it
        for e in range(E):
            beats = np.sum((l32[t] > l32[t, e]) | ((l32[t] == l32[t, e]) & (np.arange(E) < e)))
            mask[t, e] = 1.0 if beats < k else 0.0
    w = p * mask
    w = w / w.sum(axis=1, keepdims=True)

    def dense_expert(blob, F):
        lay = blob_layout(D, F)
        raw = np.asarray(blob).view(np.uint8).reshape(-1)
        sec = lambda n: raw[lay[n][0]:lay[n][0] + lay[n][1]]
        wg = _weights_bitwise(sec("gate.codes"), sec("gate.meta"), F, D, 4)
        wu = _weights_bitwise(sec("up.codes"), sec("up.meta"), F, D, 4)
        wd = _weights_bitwise(sec("down.codes"), sec("down.meta"), D, F, 4)
        pre_g = np.einsum("td,fd->tf", x, wg)
        pre_u = np.einsum("td,fd->tf", x, wu)
        act = 0.5 * pre_g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (pre_g + 0.044715 * pre_g ** 3)))
        return np.einsum("tf,df->td", act * pre_u, wd)

    out = np.zeros((T, D))
    for e in range(E):
        out += w[:, e:e + 1] * dense_expert(layer.experts[e], layer.F)
    if layer.shared is not None:
        out += dense_expert(layer.shared, layer.F_shared)
    return {"out": out, "weights": w, "logits": logits}


# --------------------------------------------------------------------------
# token -> expert permutation (prefill chunks)
# --------------------------------------------------------------------------
def permutation(ids: np.ndarray, E: int):
    """Group the (token, slot) pairs of a chunk by expert.

    counts[e]: pairs routed to e; offsets: exclusive prefix sum (E + 1
    entries); perm[p]: flat index t * k + j of the p-th pair when pairs are
    ordered by (expert, flat index); inv[t * k + j]: position of that pair.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    perm = np.empty(flat.size, dtype=np.int64)
    inv = np.empty(flat.size, dtype=np.int64)
    for i, e in enumerate(flat):
        perm[fill[e]] = i
        inv[i] = fill[e]
        fill[e] += 1
    return counts, offsets, perm, inv


# --------------------------------------------------------------------------
# per-layer LFU expert cache (streamed decode)
# --------------------------------------------------------------------------
class LFUCache:
    """Slot cache of one layer, least-frequently-used replacement.

    The pages keep 16 expert slots per layer and on a miss replace the least
    frequently used expert currently resident (stork.ai blog, "Mas inteligente
    que tu RAM"; es.news.hada.io, "Proceso de generacion de tokens").
    Readings: use counts are cumulative per expert and survive eviction; the
    victim is a resident expert the current token does not need, with the
    smallest count, ties to the least recently used, then the lowest slot;
    empty slots fill in slot order.
    """

    def __init__(self, slots: int, E: int):
        self.slots = slots
        self.count = [0] * E
        self.last = [-1] * E
        self.slot_of = [-1] * E
        self.expert_in = [-1] * slots
        self.now = 0

    def access(self, ids: Sequence[int]) -> List[Tuple[int, int, bool, int]]:
        """Serve one token's experts; returns (expert, slot, hit, evicted)."""
        ids = [int(e) for e in ids]
        if len(set(ids)) != len(ids) or len(ids) > self.slots:
            raise ValueError("ids must be distinct and fit the slots")
        for e in ids:
            self.count[e] += 1
            self.last[e] = self.now
        need = set(ids)
        events = []
        for e in ids:
            if self.slot_of[e] >= 0:
                events.append((e, self.slot_of[e], True, -1))
                continue
            empty = [s for s in range(self.slots) if self.expert_in[s] < 0]
            if empty:
                s, victim = empty[0], -1
            else:
                cands = [(self.count[v], self.last[v], s) for s, v in enumerate(self.expert_in)
                         if v not in need]
                _, _, s = min(cands)
                victim = self.expert_in[s]
                self.slot_of[victim] = -1
            self.expert_in[s] = e
            self.slot_of[e] = s
            events.append((e, s, False, victim))
        self.now += 1
        return events


class LRUCache:
    """Slot cache of one layer, least-recently-used replacement: a policy to
    compare with the pages' LFU (they report other cache policies losing to
    it: hndistilled.com, "Enfoque tecnico").  The victim is the resident
    expert that the current token does not need and whose last use is the
    oldest, ties to the lowest slot; empty slots fill in slot order.
    """

    def __init__(self, slots: int, E: int):
        self.slots = slots
        self.last_use = [-1] * E
        self.where = [-1] * E          # slot of each resident expert
        self.holder = [-1] * slots     # expert in each slot
        self.t = 0

    def access(self, ids: Sequence[int]) -> List[Tuple[int, int, bool, int]]:
        """Serve one token's experts; returns (expert, slot, hit, evicted)."""
        ids = [int(e) for e in ids]
        if len(set(ids)) != len(ids) or len(ids) > self.slots:
            raise ValueError("ids must be distinct and fit the slots")
        for e in ids:
            self.last_use[e] = self.t
        out = []
        for e in ids:
            if self.where[e] >= 0:
                out.append((e, self.where[e], True, -1))
                continue
            if -1 in self.holder:
                slot, evicted = self.holder.index(-1), -1
            else:
                slot = min((s for s in range(self.slots) if self.holder[s] not in ids),
                           key=lambda s: (self.last_use[self.holder[s]], s))
                evicted = self.holder[slot]
                self.where[evicted] = -1
            self.holder[slot] = e
            self.where[e] = slot
            out.append((e, slot, False, evicted))
        self.t += 1
        return out
