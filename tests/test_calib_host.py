"""Host-side calibration of the package (basis, Hadamard fold, C1, C2) against the oracle (no GPU)."""
import os

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


def _layer_allocation(wl):
    n = wl.n_kv_heads
    if wl.allocation[0] == "c2":
        alloc, _, _ = calib.calibrate_layer(
            [W.covariance(wl, "K", h) for h in range(n)], [W.covariance(wl, "V", h) for h in range(n)],
            lambda h, r: W.hadamard_signs(wl, "K", h, r), lambda h, r: W.hadamard_signs(wl, "V", h, r),
            wl.allocation, [W.query_covariance(wl, h) for h in range(n)])
        return alloc
    return [tuple(a) for a in wl.allocation[1]]


def test_frozen_layouts_are_the_calibration_output():
    """Each frozen layer allocation compiled into a kernel class is, head by head, what
    calibration picks for that layer (a stale line would leave the layout on the generic
    kernel), and freeze_line writes exactly that line."""
    from decode_attention_04_amd import build

    frozen = {name: (h, heads) for name, h, heads in build.frozen_layouts()}
    for wl in (W.QWEN_T128K, W.llama_t128k_c2(2.0), W.llama_t128k_c2(2.0, "joint")):
        alloc = _layer_allocation(wl)
        assert frozen[wl.name] == (1, alloc), wl.name
        line = calib.freeze_line(wl.name, alloc)
        assert line.split()[:2] == [wl.name, "1"]
        assert [tuple(int(v) for v in t.split(":")) for t in line.split()[2:]] == alloc


def test_frozen_class_generator(tmp_path):
    """Generated sources: one class per layout listing its distinct formats in order, the
    header flags, and an empty list that still yields the lookups and the dispatcher."""
    from decode_attention_04_amd import build

    srcs = build.generate([("a", 1, [(16, 4, 32, 2), (16, 4, 32, 2), (64, 3, 16, 8)]), ("b", 0, [(32, 2, 32, 2)])],
                          str(tmp_path))
    assert [os.path.basename(p) for p in srcs] == ["attend_frozen0.hip", "attend_frozen1.hip",
                                                   "attend_frozen_dispatch.hip"]
    h = (tmp_path / "attend_frozen.h").read_text()
    assert "constexpr int kFrozenClasses = 2;" in h
    assert "#define KVTC_FROZEN_CLASS0(X) X(0, 16, 4, 32, 2) X(1, 64, 3, 16, 8)" in h
    assert "return i == 0 ? 1 : i == 1 ? 0 : 1;" in h
    assert "KVTC_DEFINE_ATTEND_CLASS(frozen1, KVTC_FROZEN_CLASS1, 0)" in (tmp_path / "attend_frozen1.hip").read_text()
    srcs = build.generate([], str(tmp_path))
    assert [os.path.basename(p) for p in srcs] == ["attend_frozen_dispatch.hip"]
    assert "constexpr int kFrozenClasses = 0;" in (tmp_path / "attend_frozen.h").read_text()
    with pytest.raises(ValueError):
        bad = tmp_path / "bad.txt"
        bad.write_text("x 1 48:4:16:4\n")
        build.frozen_layouts(str(bad))


def test_static_scale_word_matches_the_oracle():
    """The product's fixed quantizer of header-free records (golden-section clip) against
    the oracle's (scanned clip, same reading), as fp16 bits, on generated heads."""
    import workloads as W
    from decode_attention_04_amd import calib
    from oracle import quantizer, transform

    wl = W.llama_t128k(0.5)
    for h in range(4):
        cov = W.covariance(wl, "K", h)
        _, vecs = transform.eigenbasis(cov)
        for r, b in ((16, 4), (32, 2), (64, 8)):
            P = transform.folded_basis(vecs, r, W.hadamard_signs(wl, "K", h, r)).astype(np.float32)
            s = float(np.sqrt(np.trace(P.astype(np.float64).T @ cov @ P.astype(np.float64)) / r))
            mu, sg = quantizer.static_scale(s, b)
            word = int(quantizer.fp16_bits(mu)) | (int(quantizer.fp16_bits(sg)) << 16)
            assert calib.static_scale_word(cov, P, b) == word, (h, r, b)


def test_nova_key_bases_match_the_oracle():
    """The product's attention-aware key bases against the oracle's: the oblique projector
    P_K Q_K^T (invariant to eigenvector signs and to the Hadamard fold), biorthogonality,
    and the coefficient variances that C1 uses."""
    from oracle import transform as T

    wl = W.llama_t128k_nova(2.0)
    for h in range(3):
        mq, sk = W.query_covariance(wl, h), W.covariance(wl, "K", h)
        w_ref, _, _ = T.nova_key_transform(mq, sk)
        for r in (16, 64):
            P, Q, lam = calib.nova_key_bases(mq, sk, r, W.hadamard_signs(wl, "K", h, r))
            Pr, Qr = T.nova_key_bases(mq, sk, r)
            assert np.allclose(P.astype(np.float64) @ Q.astype(np.float64).T, Pr @ Qr.T, atol=1e-5)
            assert np.allclose(P.astype(np.float64).T @ Q.astype(np.float64), np.eye(r), atol=1e-5)
            assert np.allclose(lam, w_ref, rtol=1e-9, atol=1e-12 * w_ref.max())


def test_pair_grouping_matches_the_oracle():
    from oracle import vq
    rng = np.random.default_rng(3)
    for n in (8, 32, 128):
        v = np.exp(rng.standard_normal(n) * 2)
        assert np.array_equal(calib.pair_order(v), vq.snake_partition(v))


def test_vq_calibration_matches_the_oracle():
    """The product's pair codebooks (all pairs at once) against the oracle's per-pair
    k-means from the same starting points: the same fp16 codewords, and calibrated heads
    whose bases reproduce the oracle's projectors."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    import harness as H
    from oracle import vq
    wl = W.llama_t128k_nova_vq(2.0)
    h = 1
    alloc, pk, qk, pv, cbk, cbv = H.oracle_calibrate_nova_vq(wl, heads=[h])
    xk = W.tokens(wl, "K", W.VQ_TRAIN_SEQ, h, 0, W.VQ_TRAIN_TOKENS).astype(np.float64)
    xv = W.tokens(wl, "V", W.VQ_TRAIN_SEQ, h, 0, W.VQ_TRAIN_TOKENS).astype(np.float64)
    # codebooks from the oracle's own bases: identical up to k-means summation order
    cb = calib.pair_codebooks(xv @ pv[0].astype(np.float64), 4, W.vq_starts(wl, "V", h, 64, 16), W.VQ_ITERS)
    assert np.abs(cb - cbv[0]).max() <= 2e-3
    assert np.mean(cb == cbv[0]) > 0.99
    # the full product calibration (eigenvector signs may differ: compare projectors and distortion)
    a, block, pv2, wk, wv = calib.calibrate_head_nova_vq(
        W.covariance(wl, "K", h), W.covariance(wl, "V", h), W.query_covariance(wl, h), xk, xv, 4,
        W.vq_starts(wl, "K", h, 64, 16), W.vq_starts(wl, "V", h, 64, 16), W.VQ_ITERS)
    assert a == alloc[0]
    p2 = block[:128 * 128].reshape(128, 128).astype(np.float64)
    q2 = block[128 * 128:].reshape(128, 128).astype(np.float64)
    assert np.allclose(p2 @ q2.T, pk[0].astype(np.float64) @ qk[0].astype(np.float64).T, atol=1e-4)
    assert np.allclose(np.abs(pv2), np.abs(pv[0]), atol=1e-5)
    assert wk.dtype == np.uint32 and wk.shape == (64 * 16,) and wv.shape == (64 * 16,)
    # the codebook words decode to codebooks whose distortion on the training values
    # is the oracle's to within a percent
    cbv2 = wv.view(np.uint16).reshape(64, 16, 2).view(np.float16).astype(np.float64)
    cv = xv @ pv2.astype(np.float64)
    cv_o = xv @ pv[0].astype(np.float64)
    d2 = np.mean((vq.decode_records(vq.encode_coords(cv, cbv2, 4), 128, 4, cbv2) - cv) ** 2)
    d1 = np.mean((vq.decode_records(vq.encode_coords(cv_o, cbv[0], 4), 128, 4, cbv[0]) - cv_o) ** 2)
    assert d2 == pytest.approx(d1, rel=0.01)
