"""Seeded synthetic inputs for the transform-coded KV cache and its decode attention.

This module is shared by the CPU oracle, the tests and the benchmark. It draws
random numbers and describes the synthetic distributions; it holds none of the
codec's arithmetic (no projection, Hadamard fold, quantizer, packing,
eigendecomposition or rank/bit allocation).

Five workloads stand in for the model workloads the pages evaluate on
(Llama-3.1-8B and Qwen2.5-7B shapes, d = 128).  No dataset or trained weight
is used; every tensor is drawn here from a seeded generator:

* keys / values of head h: x = D_o U diag(sqrt(lam)) z with z ~ N(0, I), lam_i = i^-alpha,
  U a seeded Haar-random orthogonal matrix and D_o = 20 on a few seeded
  "outlier" channels (1 elsewhere).  The analytic covariance is therefore
  D_o U diag(lam) U^T D_o, returned by ``covariance``.
* the Qwen-shaped workload replaces round(2% * d) seeded channels with
  independent heavy-tailed Student-t (nu = 3) samples scaled to 20x the
  channel's standard deviation; those rows/columns of the covariance become
  diagonal (a Student-t with nu = 3 divided by sqrt(3) has unit variance).
* queries: N(0, I) or, for the KL-ordered workload, N(0, Sigma_Q) with
  Sigma_Q = U_Q diag(i^-beta) U_Q^T per KV head.
* the random signs of the Hadamard fold are random numbers the codec draws;
  they are generated here and passed in to both sides.

Every stream is keyed by ``numpy.random.SeedSequence([workload_id, purpose, *index])``
and tokens come in fixed chunks of ``CHUNK`` so that any token range is
reproducible independently of how it is requested.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

CHUNK = 4096  # tokens per independently seeded block of keys/values

# purposes (part of the seed key)
_U, _OUTLIER, _ALPHA, _TOKENS, _QUERY, _SIGNS, _TCHAN, _QCOV, _QBETA, _VQSTART = range(1, 11)
_TENSOR = {"K": 0, "V": 1}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic workload (no codec parameters computed here)."""

    name: str
    wid: int                     # workload id, first element of every seed key
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int                 # tokens already in the cache when decoding starts
    dtype: str                   # "f32" or "f16" for keys, values and queries
    alpha: Tuple[float, float]   # spectrum exponent range (lo == hi means fixed)
    n_outliers: int = 4          # Gaussian channels scaled by outlier_scale
    outlier_scale: float = 20.0
    n_tdist: int = 0             # Student-t (nu=3) channels, scaled by outlier_scale
    query_cov: bool = False      # queries ~ N(0, Sigma_Q) instead of N(0, I)
    # allocation policy, as plain data:
    #   ("fixed", ((rk, bk, rv, bv), ...))  one tuple per KV head
    #   ("c1", budget_bits_per_dim, key_weights)  key_weights in {"mse", "kl"}; values use "mse"
    #   ("c2", budget_bits_per_dim, key_weights, "split"|"joint")  budget shared across heads
    #   ("nova", budget_bits_per_dim)  attention-aware key transform, C1 on its coefficients
    #   ("nova-vq", index_bits)  attention-aware key transform and value eigenbasis at full
    #       rank, vector-quantized coordinate pairs with index_bits bits per pair
    allocation: tuple = ()
    decode_steps: int = 1        # decode steps the workload runs (append + attend each)
    encode_tokens: int = 0       # prefill chunk encoded per sequence (0: none)
    note: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def _fixed(n_heads, rk, bk, rv, bv):
    return ("fixed", tuple((rk, bk, rv, bv) for _ in range(n_heads)))


TINY = Workload(
    name="tiny-1head-T4096", wid=0, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=128,
    context=4096, dtype="f32", alpha=(1.5, 1.5), allocation=_fixed(1, 16, 4, 32, 4),
    note="single head, fp32 keys/values, K (16,4) V (32,4)")

LLAMA_T32K = Workload(
    name="llama8b-layer-B1-T32K-2bpd", wid=1, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
    context=32768, dtype="f16", alpha=(1.0, 2.5), allocation=("c1", 2.0, "mse"),
    note="C1 at 2 bits/dim, ranks {16,32,64,128}; append 1 token + decode")


def llama_t128k(bpd: float) -> Workload:
    return Workload(
        name=f"llama8b-layer-B4-T128K-{bpd:g}bpd", wid=2, batch=4, n_q_heads=32, n_kv_heads=8,
        head_dim=128, context=131072, dtype="f16", alpha=(1.0, 2.5), query_cov=True,
        allocation=("c1", float(bpd), "kl"),
        note="C1 with attention-KL key weights from generated query variances")


def llama_t128k_c2(bpd: float, pool: str = "split") -> Workload:
    """The 128K LLaMA-shaped layer (same generated data) with the budget shared across heads:
    among the K heads and among the V heads ("split"), or among all of them ("joint")."""
    return dataclasses.replace(
        llama_t128k(bpd), name=f"llama8b-layer-B4-T128K-{bpd:g}bpd-c2" + ("" if pool == "split" else "-joint"),
        allocation=("c2", float(bpd), "kl", pool),
        note=f"C2 across the heads ({pool} K/V pools), attention-KL key weights")


def llama_t128k_nova(bpd: float) -> Workload:
    """The 128K LLaMA-shaped layer (same generated data) with the attention-aware key
    transform: its query second moment is the generated query covariance."""
    return dataclasses.replace(
        llama_t128k(bpd), name=f"llama8b-layer-B4-T128K-{bpd:g}bpd-nova", allocation=("nova", float(bpd)),
        note="keys through R_K = M_q^(1/2) E (C1 on its coefficient variances), values MSE")


def llama_t128k_nova_vq(bpd: float) -> Workload:
    """The 128K LLaMA-shaped layer (same generated data) with the attention-aware key
    transform and fixed-width vector quantization of coordinate pairs at full rank:
    2 * bpd index bits per pair of coordinates, for keys and values."""
    return dataclasses.replace(
        llama_t128k(bpd), name=f"llama8b-layer-B4-T128K-{bpd:g}bpd-nova-vq", allocation=("nova-vq", int(2 * bpd)),
        note="keys through R_K = M_q^(1/2) E, values through their eigenbasis; pairs of coefficients "
             "vector-quantized with per-pair codebooks")


# Codebook training: tokens of a sequence no workload attends over, so that the
# codebooks are fitted on data disjoint from what is encoded and measured.
VQ_TRAIN_SEQ = 1000
VQ_TRAIN_TOKENS = 4096
VQ_ITERS = 20


def vq_starts(wl: Workload, tensor: str, h: int, n_pairs: int, n_codewords: int,
              n_train: int = VQ_TRAIN_TOKENS) -> np.ndarray:
    """Starting training points of k-means: for each pair, n_codewords distinct token
    indices into the n_train training tokens (random numbers the codec draws)."""
    rng = _rng(wl.wid, _VQSTART, _TENSOR[tensor], h)
    return np.stack([rng.choice(n_train, size=n_codewords, replace=False) for _ in range(n_pairs)])


def llama_prefill(rank: int, bits: int) -> Workload:
    return Workload(
        name=f"llama8b-prefill-B16-T32K-r{rank}b{bits}", wid=3, batch=16, n_q_heads=32,
        n_kv_heads=8, head_dim=128, context=32768, dtype="f16", alpha=(1.0, 2.5),
        allocation=_fixed(8, rank, bits, rank, bits), decode_steps=64, encode_tokens=32768,
        note="kv_encode of a 32768-token chunk then 64 x (append + decode)")


QWEN_T128K = Workload(
    name="qwen7b-layer-B8-T128K-mixed", wid=4, batch=8, n_q_heads=28, n_kv_heads=4, head_dim=128,
    context=131072, dtype="f16", alpha=(1.0, 2.5), n_outliers=0, n_tdist=3,
    allocation=("fixed", ((128, 2, 128, 2), (128, 2, 128, 2), (16, 6, 16, 6), (16, 6, 16, 6))),
    encode_tokens=4096,
    note="heads 0-1 full rank r=128 b=2, heads 2-3 r=16 b=6; Student-t outlier channels")

# 256 KV heads shaped like those of the whole LLaMA-3.1-8B model (32 layers x 8 KV
# heads), for the distortion-rate characterisation: each head its own seeded
# spectrum exponent and outlier channels, as in the layer workloads.
LLAMA_256_HEADS = Workload(
    name="llama8b-256-kv-heads", wid=5, batch=1, n_q_heads=256, n_kv_heads=256, head_dim=128,
    context=4096, dtype="f16", alpha=(1.0, 2.5), allocation=("c1", 2.0, "mse"),
    note="32 layers x 8 KV heads; distortion against bits per coordinate")

ALL_BUDGETS = (0.5, 1.0, 2.0, 4.0)
C1_RANKS = (16, 32, 64, 128)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def haar_orthogonal(rng: np.random.Generator, n: int) -> np.ndarray:
    """Haar-distributed n x n orthogonal matrix (QR of a Gaussian with the sign fix)."""
    a = rng.standard_normal((n, n))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def head_alpha(wl: Workload, tensor: str, h: int) -> float:
    lo, hi = wl.alpha
    if lo == hi:
        return float(lo)
    return float(_rng(wl.wid, _ALPHA, _TENSOR[tensor], h).uniform(lo, hi))


def spectrum(wl: Workload, tensor: str, h: int) -> np.ndarray:
    """lam_i = i^-alpha, i = 1..d (descending)."""
    i = np.arange(1, wl.head_dim + 1, dtype=np.float64)
    return i ** (-head_alpha(wl, tensor, h))


def head_rotation(wl: Workload, tensor: str, h: int) -> np.ndarray:
    return haar_orthogonal(_rng(wl.wid, _U, _TENSOR[tensor], h), wl.head_dim)


def outlier_channels(wl: Workload, tensor: str, h: int) -> np.ndarray:
    rng = _rng(wl.wid, _OUTLIER, _TENSOR[tensor], h)
    return np.sort(rng.choice(wl.head_dim, size=wl.n_outliers, replace=False))


def tdist_channels(wl: Workload, tensor: str, h: int) -> np.ndarray:
    rng = _rng(wl.wid, _TCHAN, _TENSOR[tensor], h)
    return np.sort(rng.choice(wl.head_dim, size=wl.n_tdist, replace=False))


def _mixing(wl: Workload, tensor: str, h: int) -> np.ndarray:
    """L with x = L z, z ~ N(0, I) before Student-t replacement: L = D_o U diag(sqrt(lam))."""
    lam = spectrum(wl, tensor, h)
    u = head_rotation(wl, tensor, h)
    scale = np.ones(wl.head_dim)
    scale[outlier_channels(wl, tensor, h)] = wl.outlier_scale
    return (scale[:, None] * u) * np.sqrt(lam)[None, :]


def covariance(wl: Workload, tensor: str, h: int) -> np.ndarray:
    """Analytic covariance of the keys (tensor='K') or values ('V') of KV head h."""
    L = _mixing(wl, tensor, h)
    cov = L @ L.T
    if wl.n_tdist:
        ch = tdist_channels(wl, tensor, h)
        var = np.diag(cov)[ch] * wl.outlier_scale ** 2
        cov[ch, :] = 0.0
        cov[:, ch] = 0.0
        cov[ch, ch] = var
    return cov


def _chunk(wl: Workload, tensor: str, b: int, h: int, c: int, L: np.ndarray,
           tch: Optional[np.ndarray], tscale: Optional[np.ndarray]) -> np.ndarray:
    rng = _rng(wl.wid, _TOKENS, _TENSOR[tensor], b, h, c)
    z = rng.standard_normal((CHUNK, wl.head_dim))
    x = z @ L.T
    if tch is not None and len(tch):
        t = rng.standard_t(3.0, size=(CHUNK, len(tch))) / np.sqrt(3.0)
        x[:, tch] = t * tscale[None, :]
    return x


def tokens(wl: Workload, tensor: str, b: int, h: int, t0: int, n: int,
           dtype: Optional[str] = None) -> np.ndarray:
    """Keys or values of sequence b, KV head h, tokens [t0, t0+n): array [n, d].

    Returned in the workload dtype (float32 or float16) unless ``dtype='f64'``.
    """
    L = _mixing(wl, tensor, h)
    tch = tscale = None
    if wl.n_tdist:
        tch = tdist_channels(wl, tensor, h)
        tscale = np.sqrt(np.diag(L @ L.T)[tch]) * wl.outlier_scale
    out = np.empty((n, wl.head_dim), np.float64)
    c0, c1 = t0 // CHUNK, (t0 + n - 1) // CHUNK if n else t0 // CHUNK - 1
    for c in range(c0, c1 + 1):
        blk = _chunk(wl, tensor, b, h, c, L, tch, tscale)
        lo = max(t0, c * CHUNK)
        hi = min(t0 + n, (c + 1) * CHUNK)
        out[lo - t0:hi - t0] = blk[lo - c * CHUNK:hi - c * CHUNK]
    return cast(out, dtype or wl.dtype)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f64":
        return np.asarray(x, np.float64)
    if dtype == "f32":
        return np.asarray(x, np.float32)
    if dtype == "f16":
        return np.asarray(x, np.float16)
    raise ValueError(dtype)


def query_covariance(wl: Workload, h: int) -> np.ndarray:
    """Sigma_Q of the queries of KV head h (identity unless the workload draws correlated queries)."""
    d = wl.head_dim
    if not wl.query_cov:
        return np.eye(d)
    beta = float(_rng(wl.wid, _QBETA, h).uniform(0.5, 1.5))
    uq = haar_orthogonal(_rng(wl.wid, _QCOV, h), d)
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-beta)
    return (uq * lam[None, :]) @ uq.T


def queries(wl: Workload, b: int, step: int = 0, dtype: Optional[str] = None) -> np.ndarray:
    """Queries of sequence b at decode step ``step``: array [n_q_heads, d]."""
    d = wl.head_dim
    out = np.empty((wl.n_q_heads, d))
    for hq in range(wl.n_q_heads):
        h = hq // wl.group
        rng = _rng(wl.wid, _QUERY, b, hq, step)
        z = rng.standard_normal(d)
        if wl.query_cov:
            w, v = np.linalg.eigh(query_covariance(wl, h))
            out[hq] = v @ (np.sqrt(np.maximum(w, 0.0)) * z)
        else:
            out[hq] = z
    return cast(out, dtype or wl.dtype)


def hadamard_signs(wl_or_id, tensor: str, h: int, r: int) -> np.ndarray:
    """The random +-1 signs of head h's Hadamard fold (length r)."""
    wid = wl_or_id.wid if isinstance(wl_or_id, Workload) else int(wl_or_id)
    rng = _rng(wid, _SIGNS, _TENSOR[tensor], h, r)
    return np.where(rng.random(r) < 0.5, -1.0, 1.0)


def uniform_coords(seed: int, n: int, r: int) -> np.ndarray:
    """n tokens of r iid U[0,1) coordinates (float64), for quantizer-noise checks."""
    return _rng(1000, seed, n, r).random((n, r))


def random_codes(seed: int, n: int, r: int, b: int) -> np.ndarray:
    """n x r uniformly random b-bit codes (int64)."""
    return _rng(1001, seed, n, r, b).integers(0, 1 << b, size=(n, r))


def random_coords(seed: int, n: int, r: int, dtype=np.float32) -> np.ndarray:
    """n x r Gaussian coordinates with per-token random scale and offset, cast to dtype."""
    rng = _rng(1002, seed, n, r)
    scale = np.exp(rng.uniform(-4, 3, size=(n, 1)))
    off = rng.normal(size=(n, 1)) * scale
    return (rng.standard_normal((n, r)) * scale + off).astype(dtype)


def random_basis_signs(seed: int, r: int) -> np.ndarray:
    rng = _rng(1003, seed, r)
    return np.where(rng.random(r) < 0.5, -1.0, 1.0)


def random_covariance(seed: int, d: int, alpha: float = 1.5) -> np.ndarray:
    """Covariance U diag(i^-alpha) U^T with a seeded Haar U (small test heads)."""
    rng = _rng(1004, seed, d)
    u = haar_orthogonal(rng, d)
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-alpha)
    return (u * lam[None, :]) @ u.T


def random_weights(seed: int, d: int) -> np.ndarray:
    """Random positive weights sorted in decreasing order (tiny C1 heads)."""
    rng = _rng(1005, seed, d)
    return np.sort(np.exp(rng.normal(scale=2.0, size=d)))[::-1].copy()


def random_vectors(seed: int, shape: Sequence[int], dtype=np.float64) -> np.ndarray:
    return _rng(1006, seed, *shape).standard_normal(tuple(shape)).astype(dtype)


def kv_array(wl: Workload, tensor: str, t0: int, n: int, dtype: Optional[str] = None,
             threads: int = 8) -> np.ndarray:
    """Keys or values of every (sequence, KV head) for tokens [t0, t0+n): array [B, Hkv, n, d]."""
    import concurrent.futures as cf

    dt = {"f64": np.float64, "f32": np.float32, "f16": np.float16}[dtype or wl.dtype]
    out = np.empty((wl.batch, wl.n_kv_heads, n, wl.head_dim), dt)
    units = [(b, h) for b in range(wl.batch) for h in range(wl.n_kv_heads)]

    def fill(u):
        b, h = u
        out[b, h] = tokens(wl, tensor, b, h, t0, n, dtype)

    with cf.ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, units))
    return out


def query_array(wl: Workload, step: int = 0, dtype: Optional[str] = None) -> np.ndarray:
    """Queries of every sequence at decode step ``step``: array [B, Hq, d]."""
    return np.stack([queries(wl, b, step, dtype) for b in range(wl.batch)])
