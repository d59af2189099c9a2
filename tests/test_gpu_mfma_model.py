"""The matrix-core instruction's arithmetic, on which two parts of the path rest.

v_mfma_f32_16x16x32_f16 does not return the exact sum of its 32 products and its
accumulator rounded once (about half of its results differ from that).  What the path
relies on, and these tests check against exact rational sums:

* the prefill encoder's error bound E takes, per instruction, an error of at most
  k u (|C| + sum |p|) with k = 4 (u = 2^-24) for normal fp16 operands, on random
  operands over 16 binades (twice that with accumulators from far below to far
  above the products, which the encoder does not form), and on encoder-like
  operands (basis hi/lo parts against Gaussian inputs with outlier channels and
  subnormal inputs, accumulators of the size of the partial sums); products far
  below the largest are not dropped;
* the decode kernels feed b-bit codes as fp16 subnormals (code * 2^(o - 24)): their
  sums with query or probability parts are within 256 u sum |p| of exact, far inside
  the attention tolerance.

Runs one instruction per problem through libkvtc_probe.so (probe/mfma_probe.hip).
"""
import ctypes
import os
from fractions import Fraction

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
U = Fraction(1, 2 ** 24)


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    path = os.path.join(ROOT, "decode_attention_04_amd", "libkvtc_probe.so")
    lib = ctypes.CDLL(path)  # fails loudly when the probe is not built
    lib.kvtc_mfma_probe.restype = ctypes.c_int
    lib.kvtc_mfma_probe.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    return lib


def run(probe, a, b, c):
    """a [n][16][32], b [n][32][16] float16; c [n][16][16] float32 -> d (float32)."""
    n = a.shape[0]
    assert a.shape == (n, 16, 32) and b.shape == (n, 32, 16) and c.shape == (n, 16, 16)
    da = torch.from_numpy(np.ascontiguousarray(a.astype(np.float16)).view(np.int16)).cuda()
    db = torch.from_numpy(np.ascontiguousarray(b.astype(np.float16)).view(np.int16)).cuda()
    dc = torch.from_numpy(np.ascontiguousarray(c.astype(np.float32))).cuda()
    dd = torch.empty((n, 16, 16), dtype=torch.float32, device="cuda")
    rc = probe.kvtc_mfma_probe(da.data_ptr(), db.data_ptr(), dc.data_ptr(), dd.data_ptr(), n,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, f"probe launch failed ({rc})"
    torch.cuda.synchronize()
    return dd.cpu().numpy()


def spread_fp16(rng, shape, lo=-8, hi=8):
    """fp16 values with random signs, significands and exponents in [lo, hi)."""
    m = rng.uniform(1.0, 2.0, shape) * rng.choice([-1.0, 1.0], shape)
    return (m * np.exp2(rng.integers(lo, hi, shape))).astype(np.float16)


K_ENC = 4          # per-instruction factor the prefill encoder's bound E takes
K_CODES = 256      # bound for sums over fp16-subnormal code operands (decode)


def worst_ratio(a, b, c, d):
    """max over results of |D - exact| / (u (|C| + sum |p|))."""
    worst = Fraction(0)
    for p in range(a.shape[0]):
        for i in range(16):
            for j in range(16):
                prods = [Fraction(float(a[p, i, k])) * Fraction(float(b[p, k, j])) for k in range(32)]
                s = sum(prods, Fraction(float(c[p, i, j])))
                mag = sum(abs(x) for x in prods) + abs(Fraction(float(c[p, i, j])))
                if mag:
                    worst = max(worst, abs(Fraction(float(d[p, i, j])) - s) / (U * mag))
    return float(worst)


def test_sub_ulp_products_are_kept(probe):
    """One product of 1 and 31 of 2^-26 (each below half an ulp of 1): a chain of float32
    additions would return 1; the instruction keeps them (within one ulp of the exact
    sum), and every other result of the problem is within the encoder's bound."""
    rng = np.random.default_rng(7)
    a, b = spread_fp16(rng, (2, 16, 32)), spread_fp16(rng, (2, 32, 16))
    a[0, 0, :] = np.float16(2.0 ** -13)
    a[0, 0, 0] = np.float16(1.0)
    b[0, :, 0] = np.float16(2.0 ** -13)
    b[0, 0, 0] = np.float16(1.0)
    c = np.zeros((2, 16, 16), np.float32)
    d = run(probe, a, b, c)
    s = 1 + Fraction(31, 2 ** 26)
    assert d[0, 0, 0] > np.float32(1.0), "sub-ulp products dropped"
    assert abs(Fraction(float(d[0, 0, 0])) - s) <= Fraction(1, 2 ** 23), f"{d[0, 0, 0]!r} vs {float(s)!r}"
    k = worst_ratio(a, b, c, d)
    print(f"largest error / (u (|C| + sum|p|)): {k:.3f}")
    assert k <= K_ENC


@pytest.mark.parametrize("case", ["wide", "narrow", "wide-accumulator"])
def test_error_bound_random_operands(probe, case):
    """Random normal fp16 operands (16 or 2 binades) with a zero accumulator: every result
    within K_ENC u (sum |p|) of the exact value; with an accumulator drawn from 2^-40 to
    2^24, within twice that."""
    rng = np.random.default_rng({"wide": 1, "narrow": 2, "wide-accumulator": 3}[case])
    n = 8
    lo, hi = (-1, 1) if case == "narrow" else (-8, 8)
    a, b = spread_fp16(rng, (n, 16, 32), lo, hi), spread_fp16(rng, (n, 32, 16), lo, hi)
    c = np.zeros((n, 16, 16), np.float32)
    if case == "wide-accumulator":
        c = (rng.uniform(1.0, 2.0, (n, 16, 16)) * rng.choice([-1.0, 1.0], (n, 16, 16))
             * np.exp2(rng.integers(-40, 24, (n, 16, 16)))).astype(np.float32)
    k = worst_ratio(a, b, c, run(probe, a, b, c))
    print(f"{case}: largest error / (u (|C| + sum|p|)): {k:.3f}")
    # accumulators far outside the products' range are not the encoder's case (its
    # accumulators are partial sums of its own products); there the factor reached 3.8
    assert k <= (2 * K_ENC if case == "wide-accumulator" else K_ENC)


@pytest.mark.parametrize("part", ["hi", "lo"])
def test_error_bound_encoder_operands(probe, part):
    """The encoder's operands: A = fp16 hi or lo parts of an orthonormal basis scaled by
    2^8, B = fp16 Gaussian inputs with a 20x outlier channel and subnormal entries, C = a
    partial sum of the coordinate's size: within K_ENC u (|C| + sum |p|)."""
    rng = np.random.default_rng(21 if part == "hi" else 22)
    n = 8
    P = np.linalg.qr(rng.standard_normal((128, 128)))[0] * 256.0
    Ph = P.astype(np.float16)
    parts = Ph if part == "hi" else (P - Ph.astype(np.float64)).astype(np.float16)
    a = np.stack([parts[16 * (q % 8):16 * (q % 8) + 16, 32 * (q % 4):32 * (q % 4) + 32] for q in range(n)])
    x = rng.standard_normal((n, 32, 16))
    x[:, 3, :] *= 20.0
    x[:, ::5, ::3] *= 1e-4
    b = x.astype(np.float16)
    assert np.any((np.abs(b) < np.float16(2.0 ** -14)) & (b != 0)), "no subnormal inputs drawn"
    c = (rng.standard_normal((n, 16, 16)) * 30.0).astype(np.float32)
    k = worst_ratio(a, b, c, run(probe, a, b, c))
    print(f"encoder {part}: largest error / (u (|C| + sum|p|)): {k:.3f}")
    assert k <= K_ENC


@pytest.mark.parametrize("bits,wide", [(2, True), (4, True), (8, True), (4, False)])
def test_subnormal_code_operands(probe, bits, wide):
    """A holds b-bit codes at every offset o <= 10 - b of a 16-bit half, the fp16
    subnormals code * 2^(o - 24) the decode kernels build by masking record words; B
    holds fp16 operands over 18 binades (wide) or 2: sums within K_CODES u sum |p|."""
    rng = np.random.default_rng(bits + 10 * wide)
    n = 4
    codes = rng.integers(0, 2 ** bits, (n, 16, 32))
    offs = rng.integers(0, 10 - bits + 1, (n, 16, 32))
    a = (codes * np.exp2(offs - 24.0)).astype(np.float16)
    assert np.all(np.abs(a) < np.float16(2.0 ** -14)), "code operands must be fp16 subnormals"
    assert np.array_equal(a.astype(np.float64) * 2.0 ** 24 / np.exp2(offs), codes.astype(np.float64))
    b = spread_fp16(rng, (n, 32, 16), -4, 14) if wide else spread_fp16(rng, (n, 32, 16), 6, 8)
    c = np.zeros((n, 16, 16), np.float32)
    k = worst_ratio(a, b, c, run(probe, a, b, c))
    print(f"codes b={bits} {'wide' if wide else 'narrow'}: largest error / (u sum|p|): {k:.3f}")
    assert k <= K_CODES
