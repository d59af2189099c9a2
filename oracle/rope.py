"""Decode attention over keys compressed before the rotary position embedding
(oracle, float64).

Pages: KV-COBRA project page, *Results* (note under the results table): the keys of
the reported runs are compressed before the rotary position embedding (RoPE) is
applied.  The cache then holds the codes of the unrotated key, and a decode step
rotates each reconstructed key by its own position before the dot product with the
query.

Readings (the pages name RoPE but do not define it; each is the plainest one the
rest supports):

* RoPE is the rotary embedding of RoFormer (Su et al.): the head dimensions are
  taken in pairs (2i, 2i + 1), i < d/2, and the pair of a vector at position p is
  turned by the angle p * theta_i:
      (x_2i, x_2i+1) -> (x_2i cos a - x_2i+1 sin a,  x_2i sin a + x_2i+1 cos a),
  a = p * theta_i.  The inverse frequencies theta_i are an input (RoFormer's
  theta_i = base^(-2i/d) is ``default_inv_freq``; scaled variants are other inputs).
  A model that pairs dimensions (i, i + d/2) instead is the same rotation after a
  fixed permutation of the head dimensions, which the calibrated basis absorbs.
* The key of token t sits at position t (its index in the sequence's cache).
* The query arrives already rotated to its own position, as the model computes it.
* Scores: s_t = scale * q . RoPE(k_hat_t, t), with k_hat_t = P_K c_hat_K,t the
  reconstructed pre-RoPE key; softmax and values as in ``attention``.
"""
from __future__ import annotations

import numpy as np

from .attention import softmax
from .codec import decode_records, decode_records_static, record_slice


def default_inv_freq(d: int = 128, base: float = 10000.0) -> np.ndarray:
    """RoFormer's inverse frequencies theta_i = base^(-2i/d), i = 0 .. d/2 - 1."""
    return np.asarray(base, np.float64) ** (-np.arange(0, d, 2, dtype=np.float64) / d)


def rotate(x, positions, inv_freq) -> np.ndarray:
    """RoPE of the rows of x [..., T, d] at positions [T] (pairs (2i, 2i + 1))."""
    x = np.asarray(x, np.float64)
    ang = np.asarray(positions, np.float64)[:, None] * np.asarray(inv_freq, np.float64)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def attend_coords_rope(q, basis_k, ck, basis_v, cv, scale: float, positions, inv_freq) -> np.ndarray:
    """One query head over dequantized coordinates of pre-RoPE keys.

    q [d] (rotated to its own position), basis_k [d, r_K], ck [T, r_K], basis_v [d, r_V],
    cv [T, r_V], positions [T] -> o [d]."""
    k_hat = np.asarray(ck, np.float64) @ np.asarray(basis_k, np.float64).T
    s = scale * (rotate(k_hat, positions, inv_freq) @ np.asarray(q, np.float64))
    p = softmax(s)
    return np.asarray(basis_v, np.float64) @ (p @ np.asarray(cv, np.float64))


def attend_cache_rope(q, bases_k, bases_v, cache_k, cache_v, alloc, batch, capacity, T, scale, inv_freq,
                      static_k=None, static_v=None) -> np.ndarray:
    """Decode attention q [B, Hq, d] over records 0..T-1 of every head, the keys rotated
    by their positions 0..T-1 -> [B, Hq, d].  Arguments as ``attention.attend_cache``;
    inv_freq [d/2]."""
    q = np.asarray(q, np.float64)
    B, hq, d = q.shape
    hkv = len(alloc)
    g = hq // hkv
    rk, bk, rv, bv = (list(x) for x in zip(*alloc))
    fk = [static_k is not None] * hkv
    fv = [static_v is not None] * hkv
    pos = np.arange(T)
    out = np.zeros((B, hq, d))
    for b in range(B):
        for h in range(hkv):
            s0, s1, wk = record_slice(rk, bk, batch, capacity, h, b, 0, T, fk)
            v0, v1, wv = record_slice(rv, bv, batch, capacity, h, b, 0, T, fv)
            recs_k = np.asarray(cache_k[s0:s1]).reshape(T, wk)
            recs_v = np.asarray(cache_v[v0:v1]).reshape(T, wv)
            ck = decode_records(recs_k, rk[h], bk[h]) if static_k is None else \
                decode_records_static(recs_k, rk[h], bk[h], *static_k[h])
            cv = decode_records(recs_v, rv[h], bv[h]) if static_v is None else \
                decode_records_static(recs_v, rv[h], bv[h], *static_v[h])
            for i in range(g):
                out[b, h * g + i] = attend_coords_rope(q[b, h * g + i], bases_k[h], ck, bases_v[h], cv, scale, pos,
                                                       inv_freq)
    return out
