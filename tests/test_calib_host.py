"""Host-side calibration of the package (basis, Hadamard fold, C1) against the oracle (no GPU)."""
import numpy as np
import pytest

import workloads as W
from decode_attention_04_amd import calib
from oracle import allocation, transform


@pytest.mark.parametrize("n", [1, 2, 4, 16, 128])
def test_hadamard_equals_sylvester(n):
    assert np.array_equal(calib.hadamard(n), transform.sylvester_hadamard(n))


@pytest.mark.parametrize("kl", [False, True])
@pytest.mark.parametrize("r", [16, 64, 128])
def test_folded_basis_matches_oracle(r, kl):
    cov = W.random_covariance(21, 128)
    qcov = W.random_covariance(22, 128, alpha=0.8) if kl else None
    s = W.random_basis_signs(9, r)
    w1, v1 = calib.sorted_directions(cov, qcov)
    w2, v2 = transform.ordered_basis(cov, qcov)
    assert np.allclose(w1, w2, rtol=1e-10, atol=1e-15)
    p1 = calib.fold(v1, r, s).astype(np.float64)
    p2 = transform.folded_basis(v2, r, s)
    # eigenvectors are defined up to sign; compare the projector and the Gram matrix
    assert np.abs(p1 @ p1.T - p2 @ p2.T).max() < 1e-6
    assert np.abs(p1.T @ p1 - np.eye(r)).max() < 1e-6


def test_c1_matches_oracle_on_random_heads():
    for seed in range(20):
        w = W.random_weights(seed, 128)
        for bpd in (0.5, 1, 2, 4):
            budget = int(bpd * 128)
            assert calib.c1_search(w, budget, W.C1_RANKS) == allocation.c1(w, budget, W.C1_RANKS)[:2]
            assert calib.c1_search(w, budget, range(2, 129, 2)) == allocation.c1(w, budget)[:2]


def test_calibrate_head_c1_kl():
    wl = W.llama_t128k(1.0)
    a, pk, pv = calib.calibrate_head(W.covariance(wl, "K", 3), W.covariance(wl, "V", 3),
                                     lambda r: W.hadamard_signs(wl, "K", 3, r),
                                     lambda r: W.hadamard_signs(wl, "V", 3, r),
                                     wl.allocation, W.query_covariance(wl, 3))
    assert a[0] * a[1] <= 128 and a[2] * a[3] <= 128
    assert pk.shape == (128, a[0]) and pv.shape == (128, a[2]) and pk.dtype == np.float32
