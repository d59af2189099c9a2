"""Fixed-width record packing (oracle).

Pages: NOVA-KV abstract (a fixed per-token bit count is a layout
requirement); KV-COBRA project page, "Efficiency": the cache is stored as
packed b-bit codes.  Record of one token (r coordinates, b bits each):

* word 0: fp16 bits of the minimum in bits 0-15, fp16 bits of the step in bits 16-31;
* words 1 .. W-1: the codes as one little-endian bitstream -- bit k of code j
  is stream bit j*b + k, and stream bit s is bit (s mod 32) of word 1 + s // 32.
  Codes may straddle two words; unused high bits of the last word are zero.

W = 1 + ceil(r * b / 32) 32-bit words.

A header-free record (the head's quantizer fixed at calibration) is the same
record without word 0: ceil(r * b / 32) words of codes.
"""
from __future__ import annotations

import numpy as np

from .quantizer import fp16_bits, fp16_from_bits


def record_words(r: int, b: int) -> int:
    return 1 + (r * b + 31) // 32


def pack(mu, sigma, codes, b: int) -> np.ndarray:
    """Pack (mu, sigma, codes[..., r]) into records uint32[..., W]."""
    codes = np.asarray(codes, np.int64)
    r = codes.shape[-1]
    lead = codes.shape[:-1]
    if codes.min(initial=0) < 0 or codes.max(initial=0) >= (1 << b):
        raise ValueError("code out of range")
    w = record_words(r, b)
    nbits = 32 * (w - 1)
    # stream bit j*b + k  <-  bit k of code j
    bits = np.zeros(lead + (nbits,), np.uint64)
    for k in range(b):
        bits[..., np.arange(r) * b + k] = ((codes >> k) & 1).astype(np.uint64)
    words = np.zeros(lead + (w,), np.uint64)
    words[..., 0] = fp16_bits(mu) | (fp16_bits(sigma).astype(np.uint64) << np.uint64(16))
    stream = bits.reshape(lead + (w - 1, 32))
    shifts = np.arange(32, dtype=np.uint64)
    words[..., 1:] = (stream << shifts).sum(axis=-1)
    return words.astype(np.uint32)


def unpack(records, r: int, b: int):
    """Inverse of ``pack``: records uint32[..., W] -> (mu, sigma, codes[..., r])."""
    rec = np.asarray(records, np.uint32).astype(np.uint64)
    w = record_words(r, b)
    if rec.shape[-1] != w:
        raise ValueError("record width mismatch")
    lead = rec.shape[:-1]
    mu = fp16_from_bits(rec[..., 0] & np.uint64(0xFFFF))
    sigma = fp16_from_bits(rec[..., 0] >> np.uint64(16))
    shifts = np.arange(32, dtype=np.uint64)
    bits = ((rec[..., 1:, None] >> shifts) & np.uint64(1)).reshape(lead + (32 * (w - 1),))
    codes = np.zeros(lead + (r,), np.int64)
    for k in range(b):
        codes |= bits[..., np.arange(r) * b + k].astype(np.int64) << k
    return mu, sigma, codes


def padding_is_zero(records, r: int, b: int) -> bool:
    """True when every stream bit past r*b is zero."""
    rec = np.asarray(records, np.uint32).astype(np.uint64)
    used = r * b
    shifts = np.arange(32, dtype=np.uint64)
    bits = ((rec[..., 1:, None] >> shifts) & np.uint64(1)).reshape(rec.shape[:-1] + (-1,))
    return not bits[..., used:].any()


def pack_codes(codes, b: int) -> np.ndarray:
    """Header-free record: the code words of ``pack`` (its word 0 dropped)."""
    codes = np.asarray(codes, np.int64)
    z = np.zeros(codes.shape[:-1])
    return pack(z, z, codes, b)[..., 1:]


def unpack_codes(words, r: int, b: int) -> np.ndarray:
    """Inverse of ``pack_codes``: code words [..., W - 1] -> codes [..., r]."""
    words = np.asarray(words, np.uint32)
    full = np.concatenate([np.zeros(words.shape[:-1] + (1,), np.uint32), words], axis=-1)
    return unpack(full, r, b)[2]
