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

import math

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


# ---------------------------------------------------------------- one static quantizer per head
# KV-COBRA project page, "How KV-COBRA Works", Hadamard rotation: the rotation
# spreads energy evenly over the retained coordinates, so one uniform quantizer
# per head suffices; the abstract: no per-token overhead.  Readings: the header-
# free record stores codes only; the head's fixed min and step come from
# calibration.  With the random-sign Hadamard folded into the basis every retained
# coordinate of a head has the same variance s^2 = trace(P^T Sigma P) / r, and the
# range is [-kappa_b s, kappa_b s] with kappa_b the clipping that minimises the
# mean squared error of the b-bit endpoint grid for a Gaussian coordinate.


def quantize_static(c: np.ndarray, b: int, mu: float, sigma: float) -> np.ndarray:
    """Codes of c[..., r] with the head's fixed min and step: clip(rint((c - mu) / sigma), 0, 2^b - 1)."""
    if not sigma > 0:
        raise ValueError("a static step must be positive")
    levels = (1 << b) - 1
    u = (np.asarray(c, np.float64) - float(mu)) / float(sigma)
    return np.clip(np.rint(u), 0, levels).astype(np.int64)


def _cell_moment(a, b, c):
    """Integral over [a, b] of (x - c)^2 phi(x) dx for the standard normal density phi
    (arrays broadcast; a may be -inf and b +inf).

    With  int x^2 phi = Phi - x phi,  int x phi = -phi,  int phi = Phi:
    (1 + c^2)(Phi(b) - Phi(a)) - (b phi(b) - a phi(a)) + 2 c (phi(b) - phi(a)).
    """
    from scipy.special import ndtr

    a, b, c = np.broadcast_arrays(np.asarray(a, np.float64), np.asarray(b, np.float64), np.asarray(c, np.float64))

    def phi(x):
        return np.where(np.isfinite(x), np.exp(-0.5 * np.where(np.isfinite(x), x, 0.0) ** 2) / math.sqrt(2 * math.pi), 0.0)

    def xphi(x):
        return np.where(np.isfinite(x), np.where(np.isfinite(x), x, 0.0) * phi(x), 0.0)

    return (1.0 + c * c) * (ndtr(b) - ndtr(a)) - (xphi(b) - xphi(a)) + 2.0 * c * (phi(b) - phi(a))


def gaussian_uniform_mse(kappa, b: int):
    """E[(X - Q(X))^2], X ~ N(0, 1), Q the b-bit endpoint grid on [-kappa, kappa] (levels
    -kappa + k * step, step = 2 kappa / (2^b - 1), inputs outside clamped to the end
    levels); kappa may be an array."""
    kappa = np.asarray(kappa, np.float64)
    levels = (1 << b) - 1
    step = 2.0 * kappa / levels
    k = np.arange(levels + 1, dtype=np.float64)
    c = -kappa[..., None] + k * step[..., None]
    lo = np.where(k == 0, -np.inf, c - 0.5 * step[..., None])
    hi = np.where(k == levels, np.inf, c + 0.5 * step[..., None])
    return _cell_moment(lo, hi, c).sum(axis=-1)


def optimal_clip(b: int) -> float:
    """kappa_b: the clipping multiple with the smallest gaussian_uniform_mse, by a plain
    scan of [0.5, 6] in steps of 1e-2, then of the 4e-2 around the best in steps of 1e-6."""
    ks = np.arange(0.5, 6.0 + 5e-3, 1e-2)
    k0 = float(ks[int(np.argmin(gaussian_uniform_mse(ks, b)))])
    ks = np.arange(k0 - 2e-2, k0 + 2e-2 + 5e-7, 1e-6)
    return float(ks[int(np.argmin(gaussian_uniform_mse(ks, b)))])


def static_scale(s: float, b: int, kappa: float = None):
    """(mu, sigma) of a head whose coordinates have standard deviation s: mu = fp16(-kappa s),
    sigma = fp16((kappa s - mu) / (2^b - 1)) -- the per-token rule applied to the range
    [-kappa s, kappa s]."""
    if kappa is None:
        kappa = optimal_clip(b)
    mu = fp16_round(-kappa * s)
    sigma = fp16_round((kappa * s - mu) / ((1 << b) - 1))
    return float(mu), float(sigma)
