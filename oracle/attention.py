"""Decode attention over the compressed cache (oracle, float64).

Pages: KV-COBRA project page, "Efficiency": dequantization and the inverse
rotation run in one pass over packed codes with the rotation folded into the
basis; pith.science verdict on NOVA-KV (forward implications): the inverse key
transform is folded into the query.  With P_K, P_V the head's bases and c_hat
the dequantized coordinates, attention of query q over tokens t is

    q_tilde = P_K^T q,   s_t = scale * (q_tilde . c_hat_K,t),
    p = softmax(s),      o = P_V (sum_t p_t c_hat_V,t).

This equals exact softmax attention over the reconstructed keys
k_hat = P_K c_hat_K and values v_hat = P_V c_hat_V.  Query head h' reads KV head
floor(h' / g) with g = n_q_heads / n_kv_heads (contiguous GQA groups).
"""
from __future__ import annotations

import numpy as np

from .codec import decode_records, decode_records_static


def softmax(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum (float64, last axis)."""
    s = np.asarray(s, np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attend_coords(q, basis_k, ck, basis_v, cv, scale: float) -> np.ndarray:
    """One query head over dequantized coordinates.

    q [d], basis_k [d, r_K], ck [T, r_K], basis_v [d, r_V], cv [T, r_V] -> o [d].
    """
    qt = np.asarray(basis_k, np.float64).T @ np.asarray(q, np.float64)
    s = scale * (np.asarray(ck, np.float64) @ qt)
    p = softmax(s)
    ot = p @ np.asarray(cv, np.float64)
    return np.asarray(basis_v, np.float64) @ ot


def attend_head_records(qs, basis_k, rec_k, rk, bk, basis_v, rec_v, rv, bv, scale, static_k=None, static_v=None,
                        query_basis=None):
    """Query heads qs [g, d] of one KV head over its records [T, W] -> [g, d].

    static_k / static_v: the head's fixed (min, step) when its records are header-free.
    query_basis: the d x r_K basis that projects the query when it is not the encode
    basis itself (a non-orthogonal key transform: the keys are reconstructed as
    query_basis @ c^, so q . k^ = (query_basis^T q) . c^)."""
    ck = decode_records(rec_k, rk, bk) if static_k is None else decode_records_static(rec_k, rk, bk, *static_k)
    cv = decode_records(rec_v, rv, bv) if static_v is None else decode_records_static(rec_v, rv, bv, *static_v)
    qb = basis_k if query_basis is None else query_basis
    return np.stack([attend_coords(q, qb, ck, basis_v, cv, scale) for q in np.atleast_2d(qs)])


def attend_cache(q, bases_k, bases_v, cache_k, cache_v, alloc, batch, capacity, T, scale,
                 static_k=None, static_v=None, query_bases=None):
    """Full decode attention: q [B, Hq, d] over records 0..T-1 of every head -> [B, Hq, d].

    ``alloc`` lists (r_K, b_K, r_V, b_V) per KV head; ``bases_k/v`` list the
    d x r bases; ``cache_k/v`` are the flat uint32 caches in the head-major layout.
    static_k / static_v: per-head fixed (min, step) of header-free K / V records (or None).
    query_bases: per-head query-side key bases of a non-orthogonal key transform (or None).
    """
    from .codec import record_slice

    q = np.asarray(q, np.float64)
    B, hq, d = q.shape
    hkv = len(alloc)
    g = hq // hkv
    rk = [a[0] for a in alloc]
    bk = [a[1] for a in alloc]
    rv = [a[2] for a in alloc]
    bv = [a[3] for a in alloc]
    fk = [static_k is not None] * hkv
    fv = [static_v is not None] * hkv
    out = np.zeros((B, hq, d))
    for b in range(B):
        for h in range(hkv):
            s0, s1, wk = record_slice(rk, bk, batch, capacity, h, b, 0, T, fk)
            v0, v1, wv = record_slice(rv, bv, batch, capacity, h, b, 0, T, fv)
            recs_k = np.asarray(cache_k[s0:s1]).reshape(T, wk)
            recs_v = np.asarray(cache_v[v0:v1]).reshape(T, wv)
            out[b, h * g:(h + 1) * g] = attend_head_records(
                q[b, h * g:(h + 1) * g], bases_k[h], recs_k, rk[h], bk[h],
                bases_v[h], recs_v, rv[h], bv[h], scale,
                None if static_k is None else static_k[h], None if static_v is None else static_v[h],
                None if query_bases is None else query_bases[h])
    return out

