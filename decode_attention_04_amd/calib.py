"""Host-side calibration: per-head basis and (rank, bits) allocation, the inputs of the library.

KV-COBRA project page, "How KV-COBRA Works":
* Calibration -- per-head SVD of the keys; the allocator freezes each head's
  basis, rank r* and bit-width b*.  Here the SVD basis is taken as the
  eigenvectors of the head's covariance (the right singular vectors of a
  centred sample matrix).
* Hadamard rotation -- a Walsh-Hadamard transform with a fixed random sign
  flip is folded into the projection: P = E_r diag(s) H_r / sqrt(r).
* Attention-KL reordering -- direction i is weighted by sigma^2_Q,i lambda_i
  (KL) or lambda_i (MSE) and the basis is sorted by that weight before C1.
* C1, per head -- for a budget of B code bits enumerate the ranks, take
  b = min(8, floor(B / r)) (ranks with B / r < 2 are infeasible) and keep the
  smallest D(r, b) = sum_{i>r} w_i + q(b) sum_{i<=r} w_i, q(b) = 2^(-2b)/12;
  ties go to fewer bits, then the smaller rank.
* C2, across heads -- budget moves between heads until their marginal
  distortions are equal.  That condition holds at the split of the total budget
  with the smallest summed distortion, which `c2_allocate` finds exactly (a
  multiple-choice knapsack over each head's (r, b) options, solved by dynamic
  programming over the bits spent).  The K heads and the V heads form one pool
  each, or one joint pool (the abstract's joint K+V allocation).

Calibration runs once, offline, on the host (float64 numpy); the kernels take
its output as plain arrays.  The random signs are an input (drawn by the caller).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

BITS_MIN, BITS_MAX = 2, 8


def hadamard(n: int) -> np.ndarray:
    """Walsh-Hadamard matrix of order n (power of two), natural order: (-1)^popcount(i & j)."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    idx = np.arange(n, dtype=np.int64)
    x = idx[:, None] & idx[None, :]
    parity = np.zeros_like(x)
    while np.any(x):
        parity ^= x & 1
        x >>= 1
    return 1.0 - 2.0 * parity


def sorted_directions(cov: np.ndarray, query_cov: Optional[np.ndarray] = None):
    """(weights, eigenvectors as columns) sorted by decreasing weight (MSE if query_cov is None, else KL)."""
    lam, vec = np.linalg.eigh(np.asarray(cov, np.float64))
    lam, vec = lam[::-1], vec[:, ::-1]
    if query_cov is None:
        w = lam.copy()
    else:
        w = np.sum(vec * (np.asarray(query_cov, np.float64) @ vec), axis=0) * lam
    order = np.argsort(-w, kind="stable")
    return w[order], vec[:, order]


def fold(vecs: np.ndarray, r: int, signs: np.ndarray) -> np.ndarray:
    """d x r basis E_r diag(s) H_r / sqrt(r) as float32 (row-major, the library's basis layout)."""
    s = np.asarray(signs, np.float64).reshape(r)
    p = (np.asarray(vecs, np.float64)[:, :r] * s[None, :]) @ hadamard(r) / np.sqrt(r)
    return np.ascontiguousarray(p, dtype=np.float32)


def c1_search(weights: np.ndarray, budget_bits: int, ranks: Sequence[int]) -> Tuple[int, int]:
    """Per-head C1: the (rank, bits) with the smallest D(r, b) within the code-bit budget."""
    w = np.asarray(weights, np.float64)
    csum = np.concatenate([[0.0], np.cumsum(w)])
    total = csum[-1]
    best_key, best = None, None
    for r in sorted(ranks):
        b = min(BITS_MAX, int(budget_bits) // int(r))
        if b < BITS_MIN:
            continue
        head = csum[r]
        dist = (total - head) + head * (2.0 ** (-2 * b)) / 12.0
        key = (dist, r * b, r)
        if best_key is None or key < best_key:
            best_key, best = key, (int(r), int(b))
    if best is None:
        raise ValueError("no (rank, bits) fits the budget")
    return best


def c2_allocate(weights: Sequence[np.ndarray], total_bits: int,
                ranks: Sequence[int] = (16, 32, 64, 128)) -> Tuple[List[Tuple[int, int]], float]:
    """C2: one (rank, bits) per item with the smallest summed D(r, b) within ``total_bits`` code bits.

    weights: one decreasing weight vector per item.  Returns the pairs and the total
    distortion; among equal distortions the allocation spending fewer bits wins.
    """
    items = []
    for w in weights:
        w = np.asarray(w, np.float64)
        csum = np.concatenate([[0.0], np.cumsum(w)])
        rs, bs = np.meshgrid(np.array([r for r in ranks if r <= w.size], np.int64),
                             np.arange(BITS_MIN, BITS_MAX + 1, dtype=np.int64), indexing="ij")
        rs, bs = rs.reshape(-1), bs.reshape(-1)
        if rs.size == 0:
            raise ValueError("no rank fits the head dimension")
        dist = (csum[-1] - csum[rs]) + csum[rs] * np.power(2.0, -2.0 * bs) / 12.0
        items.append((rs, bs, rs * bs, dist))
    unit = int(np.gcd.reduce(np.concatenate([it[2] for it in items])))
    n = int(total_bits) // unit
    best = np.full(n + 1, np.inf)      # best[u]: least total D of the items so far spending exactly u units
    best[0] = 0.0
    picks = []
    for rs, bs, cost, dist in items:
        cu = cost // unit
        cand = np.full((cost.size, n + 1), np.inf)
        for j in range(cost.size):
            if cu[j] <= n:
                cand[j, cu[j]:] = best[:n + 1 - cu[j]] + dist[j]
        pick = np.argmin(cand, axis=0)
        best = cand[pick, np.arange(n + 1)]
        picks.append(pick)
    if not np.isfinite(best).any():
        raise ValueError("the total budget is below the smallest allocation")
    u = int(np.argmin(best))             # first minimum: the fewest units among equal totals
    total = float(best[u])
    out = []
    for (rs, bs, cost, dist), pick in zip(reversed(items), reversed(picks)):
        j = int(pick[u])
        out.append((int(rs[j]), int(bs[j])))
        u -= int(cost[j]) // unit
    return out[::-1], total


def calibrate_layer(covs_k, covs_v, signs_k_for, signs_v_for, policy, query_covs=None,
                    ranks: Sequence[int] = (16, 32, 64, 128), head_dim: int = 128):
    """Allocation and bases of every KV head of a layer under C2.

    policy: ("c2", bits_per_dim, "mse"|"kl", "split"|"joint"): a total of
    bits_per_dim * head_dim code bits per vector on average, shared among the K heads
    and among the V heads ("split") or among all of them ("joint").
    signs_k_for / signs_v_for: callables (head, r) -> +-1 vector of length r.
    Returns (allocations [(rk, bk, rv, bv), ...], bases_k, bases_v).
    """
    if policy[0] != "c2":
        raise ValueError(f"calibrate_layer takes a c2 policy, not {policy[0]}")
    n = len(covs_k)
    kl = policy[2] == "kl"
    dk = [sorted_directions(covs_k[h], query_covs[h] if kl else None) for h in range(n)]
    dv = [sorted_directions(covs_v[h]) for h in range(n)]
    per_vector = int(round(policy[1] * head_dim))
    if policy[3] == "joint":
        pairs, _ = c2_allocate([w for w, _ in dk] + [w for w, _ in dv], per_vector * 2 * n, ranks)
        ak, av = pairs[:n], pairs[n:]
    elif policy[3] == "split":
        ak, _ = c2_allocate([w for w, _ in dk], per_vector * n, ranks)
        av, _ = c2_allocate([w for w, _ in dv], per_vector * n, ranks)
    else:
        raise ValueError(f"unknown C2 pooling {policy[3]}")
    alloc = [(ak[h][0], ak[h][1], av[h][0], av[h][1]) for h in range(n)]
    bases_k = [fold(dk[h][1], ak[h][0], signs_k_for(h, ak[h][0])) for h in range(n)]
    bases_v = [fold(dv[h][1], av[h][0], signs_v_for(h, av[h][0])) for h in range(n)]
    return alloc, bases_k, bases_v


def calibrate_head(cov_k, cov_v, signs_k_for, signs_v_for, policy, query_cov=None,
                   ranks: Sequence[int] = (16, 32, 64, 128), fixed=None, head_dim: int = 128):
    """Allocation and bases of one KV head.

    policy: ("fixed", ...) with ``fixed = (rk, bk, rv, bv)``, or ("c1", bits_per_dim, "mse"|"kl").
    signs_k_for / signs_v_for: callables r -> +-1 vector of length r.
    Returns ((rk, bk, rv, bv), P_K, P_V).
    """
    wk, vk = sorted_directions(cov_k, query_cov if (policy[0] == "c1" and policy[2] == "kl") else None)
    wv, vv = sorted_directions(cov_v)
    if policy[0] == "fixed":
        rk, bk, rv, bv = fixed
    elif policy[0] == "c1":
        budget = int(round(policy[1] * head_dim))
        rk, bk = c1_search(wk, budget, ranks)
        rv, bv = c1_search(wv, budget, ranks)
    else:
        raise ValueError(f"unknown allocation policy {policy[0]}")
    return (rk, bk, rv, bv), fold(vk, rk, signs_k_for(rk)), fold(vv, rv, signs_v_for(rv))


def concat(bases: Sequence[np.ndarray]) -> np.ndarray:
    """Concatenate per-head d x r float32 bases into the library's flat basis array."""
    return np.concatenate([np.ascontiguousarray(b, np.float32).reshape(-1) for b in bases])
