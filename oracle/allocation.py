"""Per-head rank/bit allocation (oracle).

Pages: KV-COBRA project page, "How KV-COBRA Works":

* the per-head distortion D(r, b) = sum_{i > r} w_i + q(b) sum_{i <= r} w_i with
  q(b) = 2^(-2b) / 12 (w sorted in decreasing order, 1-based i);
* C1, per head: for a head budget B enumerate the even ranks r, set b from
  B / r clipped to [2, 8], keep the pair with the smallest D.

Readings: the budget counts code bits only (r * b <= B, the per-token fp16
min/step header is overhead); b = min(8, floor(B / r)) and ranks with
floor(B / r) < 2 are infeasible (raising b to 2 would exceed the budget);
ties go to the smaller D, then fewer bits r * b, then the smaller r.
"""
from __future__ import annotations

import numpy as np

from .quantizer import q_noise

B_MIN, B_MAX = 2, 8


def distortion(w, r: int, b: int) -> float:
    """D(r, b) for weights w (decreasing)."""
    w = np.asarray(w, np.float64)
    return float(w[r:].sum() + q_noise(b) * w[:r].sum())


def c1(w, budget_bits: int, ranks=None):
    """C1 search over ranks (default: every even rank up to len(w)).  Returns (r, b, D)."""
    w = np.asarray(w, np.float64)
    if ranks is None:
        ranks = range(2, len(w) + 1, 2)
    best = None
    for r in ranks:
        b = min(B_MAX, budget_bits // r)
        if b < B_MIN:
            continue
        key = (distortion(w, r, b), r * b, r)
        if best is None or key < best[0]:
            best = (key, r, b)
    if best is None:
        raise ValueError("no feasible (rank, bits) within the budget")
    return best[1], best[2], best[0][0]
