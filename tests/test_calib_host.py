"""Host-side calibration of the package (basis, Hadamard fold, C1, C2) against the oracle (no GPU)."""
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


def _spectra(wl):
    wk = [transform.ordered_basis(W.covariance(wl, "K", h), W.query_covariance(wl, h))[0] for h in range(wl.n_kv_heads)]
    wv = [transform.ordered_basis(W.covariance(wl, "V", h))[0] for h in range(wl.n_kv_heads)]
    return wk, wv


def _check_c2(ws, total, ranks):
    got, dg = calib.c2_allocate(ws, total, ranks)
    exp, de = allocation.c2(ws, total, ranks)
    assert dg == pytest.approx(de, rel=1e-9)
    assert sum(r * b for r, b in got) <= total
    assert sum(allocation.distortion(w, r, b) for w, (r, b) in zip(ws, got)) == pytest.approx(dg, rel=1e-12)
    return got, exp


def test_c2_matches_oracle_on_random_heads():
    for seed in range(6):
        ws = [W.random_weights(40 * seed + i, 128) for i in range(5)]
        for per_head in (32, 64, 128, 200, 256, 512):
            got, exp = _check_c2(ws, per_head * len(ws), W.C1_RANKS)
            assert got == exp
        got, exp = _check_c2(ws[:3], 300, (2, 8, 30, 64))   # ranks that are not multiples of 16
        assert got == exp
    with pytest.raises(ValueError):
        calib.c2_allocate([W.random_weights(1, 128)] * 3, 3 * 31, W.C1_RANKS)


@pytest.mark.parametrize("bpd", W.ALL_BUDGETS)
def test_c2_matches_oracle_on_the_llama_heads(bpd):
    wk, wv = _spectra(W.llama_t128k(bpd))
    per = int(bpd * 128)
    for ws, total in ((wk, per * 8), (wv, per * 8), (wk + wv, per * 16)):
        got, exp = _check_c2(ws, total, W.C1_RANKS)
        assert got == exp


@pytest.mark.parametrize("pool", ["split", "joint"])
def test_calibrate_layer_c2(pool):
    wl = W.llama_t128k(2.0)
    n = wl.n_kv_heads
    alloc, pk, pv = calib.calibrate_layer(
        [W.covariance(wl, "K", h) for h in range(n)], [W.covariance(wl, "V", h) for h in range(n)],
        lambda h, r: W.hadamard_signs(wl, "K", h, r), lambda h, r: W.hadamard_signs(wl, "V", h, r),
        ("c2", 2.0, "kl", pool), [W.query_covariance(wl, h) for h in range(n)])
    wk, wv = _spectra(wl)
    if pool == "split":
        ek, _ = allocation.c2(wk, 256 * n, W.C1_RANKS)
        ev, _ = allocation.c2(wv, 256 * n, W.C1_RANKS)
    else:
        e, _ = allocation.c2(wk + wv, 256 * 2 * n, W.C1_RANKS)
        ek, ev = e[:n], e[n:]
    assert alloc == [(ek[h][0], ek[h][1], ev[h][0], ev[h][1]) for h in range(n)]
    assert sum(a[0] * a[1] + a[2] * a[3] for a in alloc) <= 256 * 2 * n
    for h in range(n):
        assert pk[h].shape == (128, alloc[h][0]) and pv[h].shape == (128, alloc[h][2])
        assert np.abs(pk[h].astype(np.float64).T @ pk[h] - np.eye(alloc[h][0])).max() < 1e-5


def test_frozen_c2_kernel_class_matches_the_calibration():
    """The specialised kernel class compiled for the LLaMA-shaped C2 layout at 2 bits/dim
    lists exactly the per-head formats its calibration picks (else the layout would
    silently fall back to the generic kernel)."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(calib.__file__), "csrc", "attend_spec.h")).read()
    body = re.search(r"#define KVTC_SPEC_CLASS5\(X\)(.*)", src).group(1)
    listed = [tuple(int(v) for v in m[1:]) for m in re.findall(r"X\((\d+), (\d+), (\d+), (\d+), (\d+)\)", body)]
    wl = W.llama_t128k_c2(2.0)
    n = wl.n_kv_heads
    alloc, _, _ = calib.calibrate_layer(
        [W.covariance(wl, "K", h) for h in range(n)], [W.covariance(wl, "V", h) for h in range(n)],
        lambda h, r: W.hadamard_signs(wl, "K", h, r), lambda h, r: W.hadamard_signs(wl, "V", h, r),
        wl.allocation, [W.query_covariance(wl, h) for h in range(n)])
    assert sorted(set(alloc)) == sorted(set(listed))
