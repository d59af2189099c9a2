"""Per-token uniform b-bit scalar quantizer with fp16 min and step (oracle, float64).

Pages: KV-COBRA project page, "How KV-COBRA Works": each retained coordinate is
quantized with its head's b*-bit uniform quantizer, b in [2, 8] (C1
paragraph); the Hadamard paragraph says one uniform quantizer per head
suffices.  The record stores, per token, the quantizer's minimum and step as
fp16 followed by the codes.

Readings (where the pages are silent):
* grid: x_hat = min + code * step with step = (max - min) / (2^b - 1), the
  endpoint grid of an asymmetric min/max quantizer;
* min and step are rounded to fp16 with round-to-nearest-even, the step is
  computed from the *rounded* min, and a negative range (all coordinates
  below the rounded min) gives step 0;
* code = clip(round_half_even((c - min) / step), 0, 2^b - 1); step 0 gives
  all-zero codes.
"""
from __future__ import annotations

import numpy as np


def fp16_round(x) -> np.ndarray:
    """Round float64 values to the nearest fp16 (ties to even), returned as float64.

    numpy converts float64 to float16 directly from the double's bits with one
    rounding (no detour through float32); the tests pin this on values that
    double rounding would get wrong.
    """
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def fp16_bits(x) -> np.ndarray:
    """IEEE binary16 bit patterns (uint32) of values already exactly representable in fp16."""
    h = np.asarray(x, np.float64).astype(np.float16)
    if not np.array_equal(h.astype(np.float64), np.asarray(x, np.float64), equal_nan=True):
        raise ValueError("value not representable in fp16")
    return h.view(np.uint16).astype(np.uint32)


def fp16_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)


def quantize(c: np.ndarray, b: int):
    """Quantize coordinates c[..., r] (float64) with b bits per coordinate.

    Returns (mu, sigma, codes): mu, sigma float64 values exactly representable
    in fp16 (shape c.shape[:-1]) and codes int64 in [0, 2^b - 1].
    """
    if not 1 <= b <= 16:
        raise ValueError("bits out of range")
    c = np.asarray(c, np.float64)
    levels = (1 << b) - 1
    lo = c.min(axis=-1)
    hi = c.max(axis=-1)
    mu = fp16_round(lo)
    sigma = fp16_round(np.maximum(hi - mu, 0.0) / levels)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (c - mu[..., None]) / sigma[..., None]
    codes = np.clip(np.rint(np.where(sigma[..., None] > 0, u, 0.0)), 0, levels)
    return mu, sigma, codes.astype(np.int64)


def dequantize(mu, sigma, codes) -> np.ndarray:
    """x_hat = mu + sigma * code (float64)."""
    return np.asarray(mu, np.float64)[..., None] + np.asarray(sigma, np.float64)[..., None] * np.asarray(codes, np.float64)


def q_noise(b) -> np.ndarray:
    """High-resolution noise factor of a b-bit uniform quantizer on a unit range: q(b) = 2^(-2b) / 12.

    KV-COBRA project page, "How KV-COBRA Works", the per-head distortion D(r, b).
    """
    return np.power(2.0, -2.0 * np.asarray(b, np.float64)) / 12.0
