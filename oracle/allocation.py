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

import math

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


def options(w, ranks):
    """Every (r, b) a head can take -- r from ``ranks``, b in [2, 8] -- as (bits r*b, D(r, b), r, b)."""
    out = []
    for r in ranks:
        if r > len(w):
            continue
        for b in range(B_MIN, B_MAX + 1):
            out.append((r * b, distortion(w, r, b), r, b))
    return out


def c2(weights, total_bits: int, ranks=None):
    """C2 across heads: one (r, b) per item minimising the summed distortion within a total budget.

    Pages: KV-COBRA project page, "How KV-COBRA Works", C2 across heads (budget is
    moved between heads, C1 serving as each head's oracle, until their marginal
    distortions are equal: the water-filling condition), and the abstract (the same
    allocator applied jointly to the K and V heads).

    Reading: the allocation that condition characterises is the one with the smallest
    total distortion sum_i D_i(r_i, b_i) subject to sum_i r_i b_i <= total_bits (C1's
    budget counting: code bits only).  A head given budget B_i takes C1's pair, the
    smallest-D option with r b <= B_i, so searching over the heads' (r, b) options
    directly is the same as searching over budget splits.  The pages' damped update
    is one way to reach it; here it is computed exactly by dynamic programming over
    the bits spent, item by item.  ``weights``: one decreasing weight vector per item
    (a KV head's key or value spectrum).  Returns ([(r, b), ...], total D).
    Ties: the smaller total D, then fewer bits spent.
    """
    opts = [options(np.asarray(w, np.float64), ranks if ranks is not None else range(2, len(w) + 1, 2))
            for w in weights]
    if any(not o for o in opts):
        raise ValueError("an item has no (rank, bits) option")
    unit = 0
    for o in opts:
        for bits, _, _, _ in o:
            unit = math.gcd(unit, bits)
    n_units = int(total_bits) // unit
    # table[u] = (total D, choices) over the items so far, spending exactly u units
    table = {0: (0.0, [])}
    for o in opts:
        nxt = {}
        for spent, (dist, picks) in table.items():
            for bits, dj, r, b in o:
                u = spent + bits // unit
                if u > n_units:
                    continue
                cand = (dist + dj, picks + [(r, b)])
                if u not in nxt or cand[0] < nxt[u][0]:
                    nxt[u] = cand
        table = nxt
    if not table:
        raise ValueError("the total budget is below the smallest allocation")
    best_u = min(table, key=lambda u: (table[u][0], u))
    return table[best_u][1], table[best_u][0]
