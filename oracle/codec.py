"""Encode side of the codec and the cache layout (oracle, float64).

Pages: KV-COBRA project page, "How KV-COBRA Works", Inference: each key is
rotated and truncated with the head's basis and quantized with its head's
b*-bit quantizer; the kernel is shared by all heads and only the allocation
(rank, bits) changes per head.

Cache layout (one flat uint32 array per tensor): head-major regions, region h
holds batch x capacity records of W_h words, record (h, b, t) at word offset
sum_{h' < h} batch * capacity * W_h'  +  (b * capacity + t) * W_h.
"""
from __future__ import annotations

import numpy as np

from .packing import pack, pack_codes, record_words, unpack, unpack_codes
from .quantizer import dequantize, quantize, quantize_static


def project(x, basis) -> np.ndarray:
    """Code coordinates c = P^T x for rows x[..., d] (float64)."""
    return np.asarray(x, np.float64) @ np.asarray(basis, np.float64)


def encode_tokens(x, basis, b: int) -> np.ndarray:
    """x[n, d] -> records uint32[n, W]: project, quantize, pack."""
    c = project(x, basis)
    mu, sigma, codes = quantize(c, b)
    return pack(mu, sigma, codes, b)


def decode_records(records, r: int, b: int) -> np.ndarray:
    """records[..., W] -> dequantized coordinates[..., r] (float64)."""
    mu, sigma, codes = unpack(records, r, b)
    return dequantize(mu, sigma, codes)


def encode_tokens_static(x, basis, b: int, mu: float, sigma: float) -> np.ndarray:
    """x[n, d] -> header-free records uint32[n, W - 1] with the head's fixed min and step."""
    return pack_codes(quantize_static(project(x, basis), b, mu, sigma), b)


def decode_records_static(words, r: int, b: int, mu: float, sigma: float) -> np.ndarray:
    """Header-free records [..., W - 1] -> dequantized coordinates mu + sigma * code (float64)."""
    return float(mu) + float(sigma) * unpack_codes(words, r, b).astype(np.float64)


def width(r: int, b: int, static: bool = False) -> int:
    """Words per record: with the per-token header, or header-free."""
    return record_words(r, b) - (1 if static else 0)


def region_offsets(ranks, bits, batch: int, capacity: int, static=None) -> np.ndarray:
    """Word offset of each head's region, plus the total as the last entry (static: per-head
    flags of header-free records)."""
    st = static if static is not None else [False] * len(ranks)
    sizes = [batch * capacity * width(r, b, s) for r, b, s in zip(ranks, bits, st)]
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def record_slice(ranks, bits, batch, capacity, h, b, t0, t1, static=None):
    """(start, stop, W) word range of records t0..t1-1 of head h, sequence b."""
    off = region_offsets(ranks, bits, batch, capacity, static)
    w = width(ranks[h], bits[h], bool(static[h]) if static is not None else False)
    base = off[h] + (b * capacity) * w
    return base + t0 * w, base + t1 * w, w


def concat_bases(bases) -> np.ndarray:
    """Concatenate per-head d x r bases (row-major each) into one float32 array."""
    return np.concatenate([np.asarray(p, np.float32).reshape(-1) for p in bases])
