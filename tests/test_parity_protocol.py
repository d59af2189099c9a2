"""The parity protocol's own checks, on the CPU: the tie classifier that every GPU
encode comparison goes through accepts only off-by-one codes at a rounding tie,
and rejects the plausible mistakes (a code off by one away from a tie, off by
two, a differing header).  Records come from the oracle; the planted mistakes
are planted in copies of them."""
import numpy as np
import pytest

import harness as H
from oracle import codec, packing, quantizer


def _identity_case():
    """One token whose 16 coordinates are exactly x[:16] (P = the first 16 unit
    vectors): min 0 and max 15 give step 1, coordinate 2 sits exactly on the tie
    2.5 (round half to even: code 2), coordinate 3 at 2.3 (code 2, far from a tie)."""
    P = np.zeros((128, 16), np.float32)
    P[np.arange(16), np.arange(16)] = 1.0
    x = np.zeros((1, 128), np.float64)
    x[0, :16] = [0.0, 15.0, 2.5, 2.3, 7.0, 1.0, 3.0, 4.0, 5.0, 6.0, 8.0, 9.0, 10.0, 11.0, 12.0, 13.0]
    rec = codec.encode_tokens(x, P, 4)
    return x, P, rec


def _with_code(rec, r, b, j, code):
    mu, sg, c = packing.unpack(rec, r, b)
    c = c.copy()
    c[0, j] = code
    return packing.pack(mu, sg, c, b)


def test_identical_records_pass():
    x, P, rec = _identity_case()
    assert H.compare_records(rec.copy(), rec, 16, 4, "same", x, P) == 0.0


def test_tie_is_accepted():
    x, P, rec = _identity_case()
    assert packing.unpack(rec, 16, 4)[2][0, 2] == 2  # half to even
    got = _with_code(rec, 16, 4, 2, 3)                 # the other side of the tie
    n = H.classify_ties(x, P, *packing.unpack(rec, 16, 4)[:2], packing.unpack(got, 16, 4)[2],
                        packing.unpack(rec, 16, 4)[2], "tie")
    assert n == 1


def test_off_by_one_away_from_a_tie_is_rejected():
    x, P, rec = _identity_case()
    got = _with_code(rec, 16, 4, 3, 3)  # 2.3 rounds to 2, never to 3
    with pytest.raises(AssertionError, match="not a rounding tie"):
        H.compare_records(got, rec, 16, 4, "planted", x, P)


def test_off_by_two_is_rejected():
    x, P, rec = _identity_case()
    got = _with_code(rec, 16, 4, 2, 4)
    with pytest.raises(AssertionError, match="code 4 against 2"):
        H.compare_records(got, rec, 16, 4, "planted", x, P)


def test_header_difference_is_rejected():
    x, P, rec = _identity_case()
    got = rec.copy()
    got[0, 0] ^= 1  # last bit of the fp16 min
    with pytest.raises(AssertionError, match="headers differ"):
        H.compare_records(got, rec, 16, 4, "planted", x, P)


def test_differences_without_inputs_are_rejected():
    x, P, rec = _identity_case()
    got = _with_code(rec, 16, 4, 2, 3)
    with pytest.raises(AssertionError, match="no inputs"):
        H.compare_records(got, rec, 16, 4, "no inputs")


def test_tie_fraction_gate():
    """Classified ties still count against the 1e-5 share of codes."""
    x, P, rec = _identity_case()
    got = _with_code(rec, 16, 4, 2, 3)
    with pytest.raises(AssertionError, match="of codes differ"):
        H.compare_records(got, rec, 16, 4, "one tie in 16 codes", x, P)


@pytest.mark.parametrize("b", [2, 8])
def test_header_finite_at_the_input_norm_limit(b):
    """Inputs with ||x||_2 = 65504 (the supported limit): every coordinate of an
    orthonormal basis lies within the norm, so the fp16 min and step stay finite and
    every code is in range; adversarial tokens put the norm on the two extreme
    coordinates."""
    rng = np.random.default_rng(5)
    Q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    P = Q[:, :32]
    toks = [rng.standard_normal(128) for _ in range(8)]
    toks.append(P[:, 0] - P[:, 1])       # min and max of equal size and opposite sign
    toks.append(-P[:, 3])                # all the norm on the minimum
    toks.append(P[:, 5])                 # all the norm on the maximum
    x = np.stack([t / np.linalg.norm(t) * 65504.0 for t in toks])
    c = x @ P
    mu, sg, codes = quantizer.quantize(c, b)
    assert np.isfinite(mu).all() and np.isfinite(sg).all()
    assert (codes >= 0).all() and (codes <= (1 << b) - 1).all()
    xh = quantizer.dequantize(mu, sg, codes)
    assert np.isfinite(xh).all()
