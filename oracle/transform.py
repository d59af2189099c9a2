"""Basis of the transform coder (oracle, float64).

Pages: KV-COBRA project page, "How KV-COBRA Works": calibration takes a
per-head SVD of prefill keys; at inference each key is rotated and truncated
with H V^T; the "Hadamard rotation" paragraph folds a Walsh-Hadamard transform
with a fixed random sign flip into the projection; the "Attention-KL
reordering" paragraph weights direction i by sigma^2_Q,i * sigma^2_K,i (KL) or
by the eigenvalue lambda_i (MSE) and sorts the basis by that weight.  SPECTRA
abstract: rotate the cache into a coordinate system computed from its own
statistics.
"""
from __future__ import annotations

import numpy as np


def sylvester_hadamard(n: int) -> np.ndarray:
    """Walsh-Hadamard matrix of order n (a power of two) in Sylvester's natural order.

    H_1 = [1],  H_2m = [[H_m, H_m], [H_m, -H_m]]  (entries +-1, H H^T = n I).
    """
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def eigenbasis(cov: np.ndarray):
    """Eigenvalues (descending) and eigenvectors (columns) of a symmetric covariance.

    The right singular vectors of a centred sample matrix are the eigenvectors
    of its covariance, so this is the per-head SVD basis of the calibration
    paragraph computed from the covariance.
    """
    w, v = np.linalg.eigh(np.asarray(cov, np.float64))
    order = np.argsort(w)[::-1]
    return w[order], v[:, order]


def direction_weights(lam: np.ndarray, vecs: np.ndarray, query_cov=None) -> np.ndarray:
    """Per-direction weight: lambda_i (MSE) or sigma^2_Q,i * lambda_i (attention KL).

    sigma^2_Q,i is the query variance along key eigenvector e_i, e_i^T Sigma_Q e_i.
    """
    if query_cov is None:
        return np.asarray(lam, np.float64).copy()
    sq = np.einsum("ij,ik,kj->j", vecs, np.asarray(query_cov, np.float64), vecs)
    return sq * lam


def ordered_basis(cov: np.ndarray, query_cov=None):
    """Eigenvectors of ``cov`` sorted by decreasing direction weight, with the weights.

    Returns (weights, vectors) -- vectors are columns; stable sort keeps the
    eigenvalue order among equal weights.
    """
    lam, vecs = eigenbasis(cov)
    w = direction_weights(lam, vecs, query_cov)
    order = np.argsort(-w, kind="stable")
    return w[order], vecs[:, order]


def folded_basis(vecs: np.ndarray, r: int, signs: np.ndarray) -> np.ndarray:
    """P = E_r D_s H_r / sqrt(r): d x r basis with the random-sign Hadamard folded in.

    The code coordinates of a vector x are c = P^T x = (H_r / sqrt(r)) D_s E_r^T x:
    project onto the top-r directions, flip signs, then apply the normalised
    Hadamard.  P has orthonormal columns.
    """
    e = np.asarray(vecs, np.float64)[:, :r]
    s = np.asarray(signs, np.float64)
    if s.shape != (r,) or not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be r values in {-1, +1}")
    return (e * s[None, :]) @ sylvester_hadamard(r) / np.sqrt(r)


def basis_for_head(cov, r, signs, query_cov=None) -> np.ndarray:
    """Full calibration of one head for a given rank: ordered eigenbasis, then the fold."""
    _, vecs = ordered_basis(cov, query_cov)
    return folded_basis(vecs, r, signs)


# ---------------------------------------------------------------- attention-aware key transform (NOVA-KV)
# NOVA-KV abstract and the pith.science verdict on it (key_machinery, core_discovery):
# with M_q the second moment of the queries and S_k that of the keys, the key
# transform R_K = M_q^(1/2) E, E the eigenbasis of M_q^(1/2) S_k M_q^(1/2), is not
# orthogonal; R_K R_K^T = M_q, so coefficients r = R_K^T k turn the query-weighted
# key error into plain squared error (generalized Parseval:
# ||r - r^||^2 = (k - k^)^T M_q (k - k^)).  The inverse transform is folded into the
# query: q . k^ = (R_K^-1 q) . r^.  Readings: E sorted by decreasing eigenvalue
# (energy compaction); rank truncation keeps the first r coefficients, the key then
# reconstructed as k^ = R_K^-T [r^; 0]; a random-sign Hadamard may be folded on the
# right of both the encode basis P_K = (M_q^(1/2) E)_r and the query basis
# Q_K = (M_q^(-1/2) E)_r (it leaves P_K^T Q_K = I_r).


def psd_sqrt(m: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Symmetric square root (or its inverse) of a symmetric positive definite matrix."""
    w, v = np.linalg.eigh(np.asarray(m, np.float64))
    if w.min() <= 0:
        raise ValueError("matrix is not positive definite")
    s = np.sqrt(w)
    return (v * (1.0 / s if inverse else s)[None, :]) @ v.T


def nova_key_transform(query_moment: np.ndarray, key_moment: np.ndarray):
    """(weights, R_K, E): E the eigenvectors of M_q^(1/2) S_k M_q^(1/2) by decreasing
    eigenvalue (the weights: the coefficients' variances), R_K = M_q^(1/2) E."""
    mh = psd_sqrt(query_moment)
    w, e = eigenbasis(mh @ np.asarray(key_moment, np.float64) @ mh)
    return w, mh @ e, e


def nova_key_bases(query_moment, key_moment, r: int, signs=None):
    """(P_K, Q_K), each d x r: encode basis (M_q^(1/2) E)_r and query basis (M_q^(-1/2) E)_r,
    with the random-sign Hadamard D_s H_r / sqrt(r) folded on the right of both when
    `signs` is given."""
    _, _, e = nova_key_transform(query_moment, key_moment)
    er = e[:, :r]
    p = psd_sqrt(query_moment) @ er
    q = psd_sqrt(query_moment, inverse=True) @ er
    if signs is not None:
        s = np.asarray(signs, np.float64)
        if s.shape != (r,) or not np.all(np.abs(s) == 1.0):
            raise ValueError("signs must be r values in {-1, +1}")
        fold = s[:, None] * sylvester_hadamard(r) / np.sqrt(r)
        p, q = p @ fold, q @ fold
    return p, q
