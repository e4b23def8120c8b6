"""Shared test helpers: seeded layers on the device and parity metrics."""
from __future__ import annotations

import numpy as np

from synthetic import gen


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


# Output tolerance of the layer (fp32 output against the float64 oracle).
REL_L2 = 1e-3
MAX_ABS = 2e-2
GAP = 1e-3


def check_ids(oracle_logits: np.ndarray, ids: np.ndarray, k: int, gap: float = GAP) -> int:
    """Gap-aware check of the selected experts against the oracle's logits.

    Where the k-th / (k+1)-th logit gap exceeds ``gap`` the selected set must
    equal the oracle's exactly, and the order must match wherever adjacent
    logits differ by more than ``gap``.  Elsewhere any valid top-k is accepted:
    every chosen logit must be >= every unchosen logit - gap.  Returns the
    number of tokens that needed the tolerant rule.
    """
    T, E = oracle_logits.shape
    tolerant = 0
    for t in range(T):
        l = oracle_logits[t]
        order = sorted(range(E), key=lambda e: (-float(np.float32(l[e])), e))
        sel = [int(v) for v in ids[t]]
        assert len(set(sel)) == k and all(0 <= e < E for e in sel), (t, sel)
        kth_gap = l[order[k - 1]] - l[order[k]] if k < E else np.inf
        if kth_gap > gap:
            assert set(sel) == set(order[:k]), (t, sel, order[:k])
            for j in range(k - 1):
                if l[order[j]] - l[order[j + 1]] > gap:
                    assert sel[j] == order[j], (t, j, sel, order[:k])
        else:
            tolerant += 1
            chosen = l[sel].min()
            others = np.delete(l, sel)
            assert others.size == 0 or chosen >= others.max() - gap, (t, sel)
    return tolerant
