"""Pins of the oracle's attention over pre-RoPE keys (no GPU).

The rotary embedding is fixed against hand-worked rotations (tests/golden), an
independent complex-number form, its group laws and the relative-position property
that defines it; attention over rotated keys against textbook attention written out
with explicit keys, and against the plain oracle when every frequency is zero.
"""
import numpy as np
import pytest

import workloads as W
from conftest import read_golden
from oracle import attention, codec, rope, transform


def _floats(s):
    return np.array([float(v) for v in s.split()])


def test_rope_golden_examples():
    rows = read_golden("rope_examples.txt")
    assert len(rows) >= 5
    for x, pos, th, want in rows:
        got = rope.rotate(_floats(x)[None, :], [int(pos)], np.pi * _floats(th))[0]
        assert np.abs(got - _floats(want)).max() < 1e-14, (x, pos, th, got)


def _complex_rotate(x, positions, inv_freq):
    # pair (x_2i, x_2i+1) as the complex number x_2i + i x_2i+1, multiplied by e^(i p theta_i)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * np.outer(positions, inv_freq))
    out = np.empty(x.shape)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def test_rope_is_multiplication_by_unit_complex_numbers():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(40, 128))
    pos = rng.integers(0, 200_000, size=40)
    th = rope.default_inv_freq(128, 10000.0)
    assert np.abs(rope.rotate(x, pos, th) - _complex_rotate(x, pos, th)).max() < 1e-12


def test_rope_composes_inverts_and_keeps_pair_norms():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(17, 128))
    th = rope.default_inv_freq(128, 500000.0)
    a, b = rng.integers(-5000, 5000, size=17), rng.integers(-5000, 5000, size=17)
    assert np.abs(rope.rotate(rope.rotate(x, a, th), b, th) - rope.rotate(x, a + b, th)).max() < 1e-11
    assert np.abs(rope.rotate(rope.rotate(x, a, th), -a, th) - x).max() < 1e-12
    y = rope.rotate(x, a, th)
    assert np.allclose(y[:, 0::2] ** 2 + y[:, 1::2] ** 2, x[:, 0::2] ** 2 + x[:, 1::2] ** 2, rtol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(7)
    q, k = rng.normal(size=128), rng.normal(size=128)
    th = rope.default_inv_freq()
    for m, n in [(0, 0), (5, 3), (131071, 17), (40000, 90000)]:
        s = rope.rotate(q[None], [m], th)[0] @ rope.rotate(k[None], [n], th)[0]
        s_shift = rope.rotate(q[None], [m + 1000], th)[0] @ rope.rotate(k[None], [n + 1000], th)[0]
        s_rel = q @ rope.rotate(k[None], [n - m], th)[0]
        # angles reach 1.3e5 rad: their float64 rounding leaves ~1e-11 in the scores
        assert abs(s - s_shift) < 1e-10 and abs(s - s_rel) < 1e-10


def test_default_inverse_frequencies():
    th = rope.default_inv_freq(128, 10000.0)
    assert th.shape == (64,) and th[0] == 1.0
    assert np.isclose(th[63], 10000.0 ** (-126 / 128), rtol=1e-15)
    assert np.all(np.diff(th) < 0)
    assert np.allclose(th[1:] / th[:-1], 10000.0 ** (-2 / 128), rtol=1e-14)


def _tiny_cache(alloc, B, T, seed):
    wl = W.TINY
    bk = [transform.basis_for_head(W.random_covariance(seed + h, 128), a[0], W.random_basis_signs(seed + h, a[0]))
          for h, a in enumerate(alloc)]
    bv = [transform.basis_for_head(W.random_covariance(seed + 50 + h, 128), a[2],
                                   W.random_basis_signs(seed + 50 + h, a[2])) for h, a in enumerate(alloc)]
    rk, bitk, rv, bitv = (list(x) for x in zip(*alloc))
    ck = np.zeros(codec.region_offsets(rk, bitk, B, T)[-1], np.uint32)
    cv = np.zeros(codec.region_offsets(rv, bitv, B, T)[-1], np.uint32)
    raw_k, raw_v = [], []
    for h in range(len(alloc)):
        for b in range(B):
            k = W.tokens(wl, "K", 0, b, 0, T, dtype="f64") * (1 + h)
            v = W.tokens(wl, "V", 0, b, 0, T, dtype="f64")
            s0, s1, _ = codec.record_slice(rk, bitk, B, T, h, b, 0, T)
            ck[s0:s1] = codec.encode_tokens(k, bk[h], bitk[h]).reshape(-1)
            s0, s1, _ = codec.record_slice(rv, bitv, B, T, h, b, 0, T)
            cv[s0:s1] = codec.encode_tokens(v, bv[h], bitv[h]).reshape(-1)
            raw_k.append(k)
            raw_v.append(v)
    return bk, bv, ck, cv


def test_zero_frequencies_give_plain_attention():
    alloc = [(32, 4, 16, 8), (64, 2, 32, 4)]
    B, T, g = 2, 150, 3
    bk, bv, ck, cv = _tiny_cache(alloc, B, T, 11)
    q = np.random.default_rng(8).normal(size=(B, 2 * g, 128))
    a = rope.attend_cache_rope(q, bk, bv, ck, cv, alloc, B, T, T, 0.09, np.zeros(64))
    b = attention.attend_cache(q, bk, bv, ck, cv, alloc, B, T, T, 0.09)
    assert np.abs(a - b).max() < 1e-13


def test_rope_attention_is_textbook_attention_over_rotated_keys():
    # keys reconstructed from the records, rotated with the complex form, then
    # softmax(q . k_t * scale) weighted values, written out token by token
    alloc = [(32, 4, 16, 8), (16, 6, 64, 3)]
    B, T, g = 2, 70, 2
    bk, bv, ck, cv = _tiny_cache(alloc, B, T, 21)
    rng = np.random.default_rng(9)
    q = rng.normal(size=(B, 2 * g, 128))
    th = rope.default_inv_freq(128, 10000.0) * 3.7
    got = rope.attend_cache_rope(q, bk, bv, ck, cv, alloc, B, T, T, 0.1, th)
    rk, bitk, rv, bitv = (list(x) for x in zip(*alloc))
    for b in range(B):
        for h in range(2):
            s0, s1, wk = codec.record_slice(rk, bitk, B, T, h, b, 0, T)
            keys = codec.decode_records(ck[s0:s1].reshape(T, wk), rk[h], bitk[h]) @ bk[h].T
            s0, s1, wv = codec.record_slice(rv, bitv, B, T, h, b, 0, T)
            vals = codec.decode_records(cv[s0:s1].reshape(T, wv), rv[h], bitv[h]) @ bv[h].T
            keys = _complex_rotate(keys, np.arange(T), th)
            for i in range(g):
                qq = q[b, h * g + i]
                logits = np.array([0.1 * sum(qq[j] * kt[j] for j in range(128)) for kt in keys])
                w = np.exp(logits - logits.max())
                w /= w.sum()
                want = (w[:, None] * vals).sum(axis=0)
                assert np.abs(got[b, h * g + i] - want).max() < 1e-12 * np.abs(want).max() + 1e-14
