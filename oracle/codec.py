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

from .packing import pack, record_words, unpack
from .quantizer import dequantize, quantize


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


def region_offsets(ranks, bits, batch: int, capacity: int) -> np.ndarray:
    """Word offset of each head's region, plus the total as the last entry."""
    sizes = [batch * capacity * record_words(r, b) for r, b in zip(ranks, bits)]
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def record_slice(ranks, bits, batch, capacity, h, b, t0, t1):
    """(start, stop, W) word range of records t0..t1-1 of head h, sequence b."""
    off = region_offsets(ranks, bits, batch, capacity)
    w = record_words(ranks[h], bits[h])
    base = off[h] + (b * capacity) * w
    return base + t0 * w, base + t1 * w, w


def concat_bases(bases) -> np.ndarray:
    """Concatenate per-head d x r bases (row-major each) into one float32 array."""
    return np.concatenate([np.asarray(p, np.float32).reshape(-1) for p in bases])
