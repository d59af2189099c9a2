"""Pins of the CPU oracle to facts fixed by the pages and by mathematics (no GPU).

Each test fixes one part of the oracle against something other than its own
code: closed forms, hand-worked examples (tests/golden), brute force on tiny
inputs, or a textbook special case.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from conftest import read_golden
from oracle import allocation, attention, codec, packing, quantizer, transform


# ---------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_orthogonality_exact(n):
    h = transform.sylvester_hadamard(n)
    assert np.array_equal(h @ h.T, n * np.eye(n))


@pytest.mark.parametrize("n", [2, 8, 64, 128])
def test_hadamard_closed_form(n):
    # Sylvester's natural order: H[i, j] = (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(transform.sylvester_hadamard(n), (-1.0) ** pc)


@pytest.mark.parametrize("r", [16, 32, 64, 128])
def test_signed_normalized_hadamard_is_orthogonal(r):
    s = W.random_basis_signs(r, r)
    m = (s[:, None] * transform.sylvester_hadamard(r)) / np.sqrt(r)
    assert np.abs(m @ m.T - np.eye(r)).max() < 1e-15


# ---------------------------------------------------------------- basis
@pytest.mark.parametrize("r", [16, 32, 64, 128])
def test_folded_basis_orthonormal_and_spans_top_eigenvectors(r):
    cov = W.random_covariance(7, 128)
    lam, vecs = transform.eigenbasis(cov)
    p = transform.basis_for_head(cov, r, W.random_basis_signs(3, r))
    assert np.abs(p.T @ p - np.eye(r)).max() < 1e-13
    er = vecs[:, :r]
    assert np.abs(p @ p.T - er @ er.T).max() < 1e-12
    # eigen-decomposition really diagonalises the covariance, descending
    assert np.all(np.diff(lam) <= 1e-15)
    assert np.abs(cov @ vecs - vecs * lam[None, :]).max() < 1e-12


@pytest.mark.parametrize("r", [16, 64])
def test_truncation_error_matches_tail_eigenvalues(r):
    wl = W.TINY
    cov = W.covariance(wl, "K", 0)
    lam, _ = transform.eigenbasis(cov)
    p = transform.basis_for_head(cov, r, W.hadamard_signs(wl, "K", 0, r))
    x = W.tokens(wl, "K", 0, 0, 0, 100_000, dtype="f64")
    resid = x - (x @ p) @ p.T
    emp = (resid ** 2).sum(axis=1).mean()
    assert emp == pytest.approx(lam[r:].sum(), rel=0.02)


def test_generated_covariance_matches_samples():
    for wl in (W.TINY, W.QWEN_T128K):
        cov = W.covariance(wl, "V", 1 % wl.n_kv_heads)
        x = W.tokens(wl, "V", 0, 1 % wl.n_kv_heads, 0, 60_000, dtype="f64")
        emp = x.T @ x / len(x)
        scale = np.sqrt(np.outer(np.diag(cov), np.diag(cov)))
        assert np.abs(emp - cov).max() / scale.max() < 0.05


def test_kl_weights_use_query_variance_along_key_directions():
    cov = W.random_covariance(11, 16)
    qcov = W.random_covariance(12, 16, alpha=0.7)
    lam, vecs = transform.eigenbasis(cov)
    w = transform.direction_weights(lam, vecs, qcov)
    # sigma^2_Q,i is the variance of e_i . q, checked by sampling q ~ N(0, Sigma_Q)
    rng = np.random.default_rng(0)
    q = rng.multivariate_normal(np.zeros(16), qcov, size=200_000)
    sq = ((q @ vecs) ** 2).mean(axis=0)
    assert np.allclose(w, sq * lam, rtol=0.03)
    ws, vs = transform.ordered_basis(cov, qcov)
    assert np.all(np.diff(ws) <= 0)
    assert np.allclose(transform.direction_weights(lam, vecs), lam)


# ---------------------------------------------------------------- fp16 rounding
def test_fp16_round_is_single_rounding_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -10
    mid = one + ulp / 2  # midpoint between 1 and 1 + 2^-10
    assert quantizer.fp16_round(mid) == 1.0                     # tie -> even (1.0)
    assert quantizer.fp16_round(mid + 2.0 ** -40) == 1.0 + ulp  # above midpoint by less than a float32 ulp
    assert quantizer.fp16_round(mid - 2.0 ** -40) == 1.0
    mid2 = one + 1.5 * ulp                                       # tie between odd and even -> even (1 + 2 ulp)
    assert quantizer.fp16_round(mid2) == 1.0 + 2 * ulp
    # subnormals: spacing 2^-24
    assert quantizer.fp16_round(2.5 * 2.0 ** -24) == 2 * 2.0 ** -24
    assert quantizer.fp16_round(2.5 * 2.0 ** -24 + 2.0 ** -60) == 3 * 2.0 ** -24
    # bit patterns
    assert int(quantizer.fp16_bits(1.0)) == 0x3C00
    assert int(quantizer.fp16_bits(-2.0)) == 0xC000
    assert int(quantizer.fp16_bits(2.0 ** -24)) == 0x0001


# ---------------------------------------------------------------- quantizer
def test_quantizer_golden_examples():
    rows = read_golden("quantizer_examples.txt")
    assert len(rows) >= 9
    for b, coords, mu, sigma, codes in rows:
        c = np.array([float(v) for v in coords.split()])
        m, s, k = quantizer.quantize(c, int(b))
        assert m == float(mu), (coords, m)
        assert s == float(sigma), (coords, s)
        assert k.tolist() == [int(v) for v in codes.split()], (coords, k)


def test_q_of_b_matches_textbook_uniform_quantizer():
    # textbook b-bit quantizer on U[0,1): 2^b cells of width 2^-b, reconstruction at cell midpoints
    x = W.uniform_coords(1, 400_000, 1)[:, 0]
    for b in (2, 4, 8):
        cells = np.floor(x * 2 ** b)
        xhat = (cells + 0.5) / 2 ** b
        mse = ((x - xhat) ** 2).mean()
        assert mse / quantizer.q_noise(b) == pytest.approx(1.0, abs=0.01)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_deployed_quantizer_noise_closed_form(b):
    r = 32
    n = 100_000
    x = W.uniform_coords(2, n, r)
    mu, sigma, codes = quantizer.quantize(x, b)
    xhat = quantizer.dequantize(mu, sigma, codes)
    mse = ((x - xhat) ** 2).mean()
    L = 2 ** b
    # interior points uniform on [min, max] (error uniform over one step), the two
    # extremes reproduced; range of r uniforms ~ Beta(r-1, 2): E[R^2] = (r-1) r / ((r+1)(r+2))
    expect = quantizer.q_noise(b) * (L / (L - 1)) ** 2 * ((r - 2) / r) * ((r - 1) * r / ((r + 1) * (r + 2)))
    assert mse / expect == pytest.approx(1.0, abs=0.02)


def test_quantizer_error_bound_and_range():
    x = W.random_coords(5, 3000, 64).astype(np.float64)
    for b in range(2, 9):
        mu, sigma, codes = quantizer.quantize(x, b)
        xhat = quantizer.dequantize(mu, sigma, codes)
        assert codes.min() >= 0 and codes.max() <= 2 ** b - 1
        # every coordinate inside [mu, mu + (2^b-1) sigma] is within half a step
        top = mu + (2 ** b - 1) * sigma
        inside = (x >= mu[:, None]) & (x <= top[:, None])
        err = np.abs(x - xhat)
        half = np.broadcast_to(sigma[:, None] / 2 * (1 + 1e-12), err.shape)
        assert np.all(err[inside] <= half[inside])
        # only the extremes can fall outside (fp16 rounding of min and step); they stay close
        assert inside.mean() > 0.95
        slack = np.broadcast_to((sigma + 2.0 ** -10 * (np.abs(mu) + (2 ** b - 1) * sigma))[:, None], err.shape)
        assert np.all(err[~inside] <= slack[~inside])
        # the fp16 header is exactly what is stored
        assert np.array_equal(quantizer.fp16_round(mu), mu)
        assert np.array_equal(quantizer.fp16_round(sigma), sigma)


# ---------------------------------------------------------------- packing
def test_pack_golden_examples():
    for r, b, mu, sigma, codes, words in read_golden("pack_examples.txt"):
        r, b = int(r), int(b)
        c = np.array([int(v) for v in codes.split()])
        assert len(c) == r
        rec = packing.pack(np.array(float(mu)), np.array(float(sigma)), c, b)
        want = [int(w, 16) for w in words.split()]
        assert len(want) == packing.record_words(r, b)
        assert [int(v) for v in rec] == want


def _bigint_pack(codes, b, w):
    """Independent packer: the code stream as one Python integer, cut into 32-bit words."""
    acc = 0
    for j, c in enumerate(codes):
        acc |= int(c) << (j * b)
    return [(acc >> (32 * i)) & 0xFFFFFFFF for i in range(w - 1)]


@pytest.mark.parametrize("r,b", list(itertools.product([16, 32, 64, 128], range(2, 9))))
def test_pack_matches_bigint_and_round_trips(r, b):
    codes = W.random_codes(r * 10 + b, 40, r, b)
    x = W.random_coords(b, 40, r).astype(np.float64)
    mu, sigma, _ = quantizer.quantize(x, b)
    rec = packing.pack(mu, sigma, codes, b)
    w = packing.record_words(r, b)
    assert rec.shape == (40, w)
    for t in range(40):
        assert rec[t, 1:].tolist() == _bigint_pack(codes[t], b, w)
    m2, s2, c2 = packing.unpack(rec, r, b)
    assert np.array_equal(m2, mu) and np.array_equal(s2, sigma) and np.array_equal(c2, codes)
    assert packing.padding_is_zero(rec, r, b)


def test_record_words():
    assert packing.record_words(16, 4) == 3
    assert packing.record_words(32, 4) == 5
    assert packing.record_words(128, 2) == 9
    assert packing.record_words(16, 6) == 4
    assert packing.record_words(128, 8) == 33


# ---------------------------------------------------------------- attention
def _textbook(q, k, v, scale):
    # softmax(q . k_t * scale) weighted sum of v_t, written out from the definition
    logits = np.array([scale * sum(qi * ki for qi, ki in zip(q, kt)) for kt in k])
    w = np.exp(logits - logits.max())
    w = w / w.sum()
    return (w[:, None] * v).sum(axis=0)


def test_full_rank_unquantized_reproduces_exact_attention():
    d, T = 128, 300
    wl = W.TINY
    cov = W.covariance(wl, "K", 0)
    pk = transform.basis_for_head(cov, d, W.hadamard_signs(wl, "K", 0, d))
    pv = transform.basis_for_head(W.covariance(wl, "V", 0), d, W.hadamard_signs(wl, "V", 0, d))
    k = W.tokens(wl, "K", 0, 0, 0, T, dtype="f64")
    v = W.tokens(wl, "V", 0, 0, 0, T, dtype="f64")
    q = W.random_vectors(1, (d,))
    scale = 1 / np.sqrt(d)
    o = attention.attend_coords(q, pk, codec.project(k, pk), pv, codec.project(v, pv), scale)
    ref = _textbook(q, k, v, scale)
    assert np.abs(o - ref).max() / np.abs(ref).max() < 1e-12
    # scores themselves: (P^T q).(P^T k) = q.k
    s1 = codec.project(k, pk) @ (pk.T @ q)
    assert np.abs(s1 - k @ q).max() / np.abs(k @ q).max() < 1e-12


def test_attention_invariants():
    rng = np.random.default_rng(3)
    d, T, r = 128, 257, 32
    pk = transform.folded_basis(transform.eigenbasis(W.random_covariance(1, d))[1], r, W.random_basis_signs(1, r))
    pv = transform.folded_basis(transform.eigenbasis(W.random_covariance(2, d))[1], r, W.random_basis_signs(2, r))
    ck = rng.normal(size=(T, r))
    cv = rng.normal(size=(T, r))
    q = rng.normal(size=d)
    o = attention.attend_coords(q, pk, ck, pv, cv, 0.1)
    perm = rng.permutation(T)
    assert np.allclose(attention.attend_coords(q, pk, ck[perm], pv, cv[perm], 0.1), o, rtol=1e-13, atol=1e-15)
    # a single token returns its own value
    assert np.allclose(attention.attend_coords(q, pk, ck[:1], pv, cv[:1], 0.1), pv @ cv[0])
    # adding a constant to every score leaves the output unchanged (shift q along a direction
    # orthogonal to nothing is hard; instead duplicate every token: weights unchanged)
    o2 = attention.attend_coords(q, pk, np.vstack([ck, ck]), pv, np.vstack([cv, cv]), 0.1)
    assert np.allclose(o2, o, rtol=1e-12)


def test_gqa_head_equals_single_head_on_its_kv_head():
    wl = W.TINY
    d, T = 128, 64
    alloc = [(16, 4, 32, 4), (32, 8, 16, 2)]
    B, cap = 2, 64
    g = 3
    bases_k, bases_v, caches_k, caches_v = [], [], [], []
    rk, bk, rv, bv = zip(*alloc)
    ck_flat = np.zeros(codec.region_offsets(rk, bk, B, cap)[-1], np.uint32)
    cv_flat = np.zeros(codec.region_offsets(rv, bv, B, cap)[-1], np.uint32)
    for h, (a, b1, c, b2) in enumerate(alloc):
        pk = transform.basis_for_head(W.random_covariance(10 + h, d), a, W.random_basis_signs(h, a)).astype(np.float32)
        pv = transform.basis_for_head(W.random_covariance(20 + h, d), c, W.random_basis_signs(h + 5, c)).astype(np.float32)
        bases_k.append(pk)
        bases_v.append(pv)
        for b in range(B):
            k = W.tokens(wl, "K", b, 0, 0, T, dtype="f64") + h
            v = W.tokens(wl, "V", b, 0, 0, T, dtype="f64") - h
            s0, s1, _ = codec.record_slice(rk, bk, B, cap, h, b, 0, T)
            ck_flat[s0:s1] = codec.encode_tokens(k, pk, b1).reshape(-1)
            s0, s1, _ = codec.record_slice(rv, bv, B, cap, h, b, 0, T)
            cv_flat[s0:s1] = codec.encode_tokens(v, pv, b2).reshape(-1)
    q = W.random_vectors(4, (B, 2 * g, d))
    out = attention.attend_cache(q, bases_k, bases_v, ck_flat, cv_flat, alloc, B, cap, T, 0.088)
    for b in range(B):
        for hq in range(2 * g):
            h = hq // g
            s0, s1, wk = codec.record_slice(rk, bk, B, cap, h, b, 0, T)
            t0, t1, wv = codec.record_slice(rv, bv, B, cap, h, b, 0, T)
            kh = codec.decode_records(ck_flat[s0:s1].reshape(T, wk), rk[h], bk[h]) @ bases_k[h].astype(np.float64).T
            vh = codec.decode_records(cv_flat[t0:t1].reshape(T, wv), rv[h], bv[h]) @ bases_v[h].astype(np.float64).T
            ref = _textbook(q[b, hq], kh, vh, 0.088)
            assert np.abs(out[b, hq] - ref).max() <= 1e-12 * np.abs(ref).max()


# ---------------------------------------------------------------- allocation
def test_distortion_golden():
    for w, r, b, frac in read_golden("distortion_examples.txt"):
        wv = [float(v) for v in w.split()]
        num, den = frac.split("/")
        assert allocation.distortion(wv, int(r), int(b)) == pytest.approx(float(Fraction(int(num), int(den))), rel=1e-15)


def _brute_force(w, budget, ranks):
    d = len(w)
    best = None
    for r in ranks:
        for b in range(2, 9):
            if r * b > budget:
                continue
            tail = sum(w[r:])
            head = sum(w[:r])
            dist = tail + head / (12 * 4 ** b)
            key = (dist, r * b, r)
            if best is None or key < best[0]:
                best = (key, r, b)
    return best


@pytest.mark.parametrize("d", [8, 16])
def test_c1_equals_brute_force(d):
    for seed in range(12):
        w = W.random_weights(seed * 31 + d, d)
        for ranks in (None, [r for r in (2, 4, 8, 16) if r <= d]):
            rr = list(range(2, d + 1, 2)) if ranks is None else ranks
            for budget in range(0, 8 * d + 1):
                bf = _brute_force(list(w), budget, rr)
                if bf is None:
                    with pytest.raises(ValueError):
                        allocation.c1(w, budget, ranks)
                    continue
                r, b, dist = allocation.c1(w, budget, ranks)
                assert (r, b) == (bf[1], bf[2]), (seed, budget)
                assert dist == pytest.approx(bf[0][0], rel=1e-12)


def test_c1_on_generated_heads_uses_the_budget():
    wl = W.LLAMA_T32K
    for h in range(wl.n_kv_heads):
        lam, _ = transform.eigenbasis(W.covariance(wl, "K", h))
        r, b, _ = allocation.c1(lam, 256, W.C1_RANKS)
        assert r * b <= 256 and (r, b) in {(16, 8), (32, 8), (64, 4), (128, 2)}


def _c2_brute_force(ws, total, ranks):
    """Every combination of the items' (r, b) options: the least summed distortion within the bits."""
    opts = [[(r, b) for r in ranks if r <= len(w) for b in range(2, 9)] for w in ws]
    best = None
    for combo in itertools.product(*opts):
        bits = sum(r * b for r, b in combo)
        if bits > total:
            continue
        dist = sum(sum(w[r:]) + sum(w[:r]) / (12 * 4 ** b) for w, (r, b) in zip(ws, combo))
        if best is None or (dist, bits) < best[0]:
            best = ((dist, bits), list(combo))
    return best


def test_c2_equals_brute_force():
    ranks = (2, 4, 8)
    for seed in range(3):
        ws = [list(W.random_weights(seed * 7 + i, 8)) for i in range(3)]
        for total in range(0, 3 * 64 + 1, 5):
            bf = _c2_brute_force(ws, total, ranks)
            if bf is None:
                with pytest.raises(ValueError):
                    allocation.c2(ws, total, ranks)
                continue
            picks, dist = allocation.c2(ws, total, ranks)
            assert picks == bf[1], (seed, total)
            assert dist == pytest.approx(bf[0][0], rel=1e-12)


def test_c2_of_one_head_is_c1():
    for seed in range(8):
        w = W.random_weights(100 + seed, 128)
        for budget in (32, 64, 100, 128, 256, 300, 512, 1024):
            r, b, d1 = allocation.c1(w, budget, W.C1_RANKS)
            picks, d2 = allocation.c2([w], budget, W.C1_RANKS)
            assert picks == [(r, b)] and d2 == pytest.approx(d1, rel=1e-15)


def test_c2_lagrangian_allocations_are_optimal():
    """Everett's theorem: the choice minimising sum_i D_i + mu * bits_i, made item by
    item, has the least total D among all allocations spending no more bits than it."""
    for seed in range(4):
        ws = [W.random_weights(200 + 10 * seed + i, 128) for i in range(6)]
        for mu in (1e-5, 1e-4, 1e-3, 1e-2):
            combo, bits, dist = [], 0, 0.0
            for w in ws:
                cands = [(allocation.distortion(w, r, b) + mu * r * b, r * b, r, b)
                         for r in W.C1_RANKS for b in range(2, 9)]
                _, cb, r, b = min(cands)
                combo.append((r, b))
                bits += cb
                dist += allocation.distortion(w, r, b)
            picks, d2 = allocation.c2(ws, bits, W.C1_RANKS)
            assert d2 == pytest.approx(dist, rel=1e-12), (seed, mu)


def test_c2_monotone_in_budget_and_no_worse_than_uniform_c1():
    ws = [W.random_weights(300 + i, 128) for i in range(8)]
    prev = None
    for per_head in (32, 64, 96, 128, 192, 256, 384, 512):
        picks, dist = allocation.c2(ws, per_head * len(ws), W.C1_RANKS)
        assert sum(r * b for r, b in picks) <= per_head * len(ws)
        uniform = sum(allocation.c1(w, per_head, W.C1_RANKS)[2] for w in ws)
        assert dist <= uniform * (1 + 1e-12)
        if prev is not None:
            assert dist <= prev * (1 + 1e-12)
        prev = dist


# ---------------------------------------------------------------- layout
def test_region_offsets_and_record_slices():
    rk, bk = [16, 128, 16], [4, 2, 6]
    off = codec.region_offsets(rk, bk, 2, 8)
    assert off.tolist() == [0, 2 * 8 * 3, 2 * 8 * 3 + 2 * 8 * 9, 2 * 8 * 3 + 2 * 8 * 9 + 2 * 8 * 4]
    s0, s1, w = codec.record_slice(rk, bk, 2, 8, 1, 1, 2, 5)
    assert w == 9 and s0 == 48 + (1 * 8 + 2) * 9 and s1 == s0 + 3 * 9


# ------------------------------------------------------------------ header-free records (one static quantizer per head)
def test_static_quantizer_hand_worked_example():
    """min 0, step 0.5, b = 2: (c - min) / step = 0, 0.5, 1, 2, 2.4, -0.2, 7 -> rint (half to
    even) 0, 0, 1, 2, 2, -0, 7 -> clamped to [0, 3]: 0, 0, 1, 2, 2, 0, 3."""
    c = np.array([0.0, 0.25, 0.5, 1.0, 1.2, -0.1, 3.5])
    assert quantizer.quantize_static(c, 2, 0.0, 0.5).tolist() == [0, 0, 1, 2, 2, 0, 3]


@pytest.mark.parametrize("b", [2, 4, 8])
def test_static_quantizer_noise_on_its_range_is_step_squared_over_12(b):
    """Inputs uniform over the grid's span [min, min + (2^b - 1) step): every error is
    uniform over half a step or a whole cell, so E[MSE] = step^2 / 12 exactly (step 2^-b,
    exact in fp16)."""
    rng = np.random.default_rng(b)
    step = 2.0 ** -b
    c = rng.random(1_000_000) * ((1 << b) - 1) * step
    codes = quantizer.quantize_static(c, b, 0.0, step)
    mse = np.mean((c - step * codes) ** 2)
    assert abs(mse / (step * step / 12.0) - 1.0) < 0.01


@pytest.mark.parametrize("b", range(2, 9))
def test_gaussian_uniform_mse_closed_form_matches_monte_carlo(b):
    """The closed form of the clamped endpoint grid's error on N(0, 1) against the
    mean squared error of quantize_static on 2e6 samples, at the optimal clip and at
    half and twice it."""
    rng = np.random.default_rng(100 + b)
    x = rng.standard_normal(2_000_000)
    L = (1 << b) - 1
    k_opt = quantizer.optimal_clip(b)
    for k in (k_opt, 0.5 * k_opt, 2.0 * k_opt):
        step = 2.0 * k / L
        xh = -k + step * quantizer.quantize_static(x, b, -k, step)
        mc = np.mean((x - xh) ** 2)
        assert abs(mc / float(quantizer.gaussian_uniform_mse(k, b)) - 1.0) < 0.01


def test_optimal_clip_is_a_minimum_and_grows_with_bits():
    prev_k, prev_d = 0.0, np.inf
    for b in range(2, 9):
        k = quantizer.optimal_clip(b)
        d = float(quantizer.gaussian_uniform_mse(k, b))
        for delta in (1e-3, 1e-2, 1e-1):
            assert d <= float(quantizer.gaussian_uniform_mse(k + delta, b))
            assert d <= float(quantizer.gaussian_uniform_mse(k - delta, b))
        assert k > prev_k and d < prev_d
        prev_k, prev_d = k, d
    # fine grids: the error splits into the granular step^2 / 12 inside the range and
    # the overload 2 int_kappa^inf (x - kappa)^2 phi = 2 ((1 + k^2) Q(k) - k phi(k))
    from scipy.special import ndtr
    k8 = quantizer.optimal_clip(8)
    step = 2 * k8 / 255
    tail = 1.0 - ndtr(k8)
    dens = np.exp(-k8 * k8 / 2) / np.sqrt(2 * np.pi)
    overload = 2 * ((1 + k8 * k8) * tail - k8 * dens)
    granular = step * step / 12 * (1 - 2 * tail)
    d8 = float(quantizer.gaussian_uniform_mse(k8, 8))
    assert abs((granular + overload) / d8 - 1.0) < 0.01


@pytest.mark.parametrize("r", [16, 64])
def test_hadamard_fold_equalises_coordinate_variances(r):
    """With the random-sign Hadamard folded in, every retained coordinate of a head
    has the same variance trace(P^T Sigma P) / r (the mean of the retained
    eigenvalues): one static quantizer per head fits all of them."""
    cov = W.random_covariance(7, 128)
    lam, vecs = transform.eigenbasis(cov)
    P = transform.folded_basis(vecs, r, W.random_basis_signs(3, r))
    var = np.diag(P.T @ cov @ P)
    assert np.allclose(var, lam[:r].mean(), rtol=1e-12, atol=0)


def test_static_scale_uses_the_clipped_range():
    s, b = 0.75, 3
    k = quantizer.optimal_clip(b)
    mu, sg = quantizer.static_scale(s, b)
    assert mu == float(quantizer.fp16_round(-k * s))
    assert sg == float(quantizer.fp16_round((k * s - mu) / 7))
    assert quantizer.fp16_bits(mu) is not None and quantizer.fp16_bits(sg) is not None


@pytest.mark.parametrize("r", [16, 32, 64, 128])
@pytest.mark.parametrize("b", range(2, 9))
def test_header_free_records_round_trip(r, b):
    codes = W.random_codes(r * 10 + b, 50, r, b)
    words = packing.pack_codes(codes, b)
    assert words.shape == (50, packing.record_words(r, b) - 1)
    assert np.array_equal(words, packing.pack(np.zeros(50), np.zeros(50), codes, b)[:, 1:])
    assert np.array_equal(packing.unpack_codes(words, r, b), codes)


def test_header_free_attention_on_exact_grid_is_textbook_attention():
    """Full rank, identity basis, coordinates on the static grid: the header-free cache
    holds the keys and values exactly, and decode attention over it equals textbook
    softmax(q K^T / sqrt(d)) V computed directly."""
    rng = np.random.default_rng(11)
    T, d, b = 300, 128, 4
    mu, sg = -2.0, 0.25
    P = np.eye(d)
    k = mu + sg * rng.integers(0, 16, (T, d))
    v = mu + sg * rng.integers(0, 16, (T, d))
    q = rng.standard_normal((2, d))
    rk = codec.encode_tokens_static(k, P, b, mu, sg)
    rv = codec.encode_tokens_static(v, P, b, mu, sg)
    got = attention.attend_head_records(q, P, rk, d, b, P, rv, d, b, 1 / np.sqrt(d), (mu, sg), (mu, sg))
    s = q @ k.T / np.sqrt(d)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ v
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_header_free_region_offsets():
    ranks, bits = [16, 64], [4, 4]
    off = codec.region_offsets(ranks, bits, 2, 10, [True, False])
    assert off.tolist() == [0, 2 * 10 * 2, 2 * 10 * 2 + 2 * 10 * 9]
    s0, s1, w = codec.record_slice(ranks, bits, 2, 10, 0, 1, 3, 5, [True, False])
    assert (s0, s1, w) == (10 * 2 + 3 * 2, 10 * 2 + 5 * 2, 2)


# ------------------------------------------------------------------ distortion against bits
@pytest.mark.parametrize("b", [6, 7, 8])
def test_quantization_noise_is_step_squared_over_12_at_high_resolution(b):
    """The per-coordinate quantization noise of the deployed quantizer on a generated
    head at full rank follows the high-resolution form behind q(b): for fine grids each
    coordinate's error is uniform over one step, so sum_j (c_j - c^_j)^2 averages
    r step_t^2 / 12 with each token's own step (within 2%)."""
    wl = W.LLAMA_256_HEADS
    x = W.tokens(wl, "K", 0, 17, 0, 4096).astype(np.float64)
    _, vecs = transform.ordered_basis(W.covariance(wl, "K", 17))
    P = transform.folded_basis(vecs, 128, W.hadamard_signs(wl, "K", 17, 128))
    c = x @ P
    mu, sg, codes = quantizer.quantize(c, b)
    noise = ((c - quantizer.dequantize(mu, sg, codes)) ** 2).sum(axis=1).mean()
    assert abs(noise / (128 * np.mean(sg ** 2) / 12) - 1.0) < 0.02


def test_full_rank_distortion_falls_by_about_four_per_bit():
    """Full rank removes the truncation term of D(r, b), and the quantization distortion
    falls by 2^2 per added bit in the q(b) = 2^(-2b) / 12 model; the deployed endpoint grid
    has step = range / (2^b - 1), so with the per-token range fixed the ratio
    D(b) / D(b + 1) is ((2^(b+1) - 1) / (2^b - 1))^2 = 4 ((2^(b+1) - 1) / (2 (2^b - 1)))^2,
    which tends to 4 from above (5.44 at b = 2): the measured ratios lie in [4, that]
    up to 3%."""
    wl = W.LLAMA_256_HEADS
    x = W.tokens(wl, "V", 0, 40, 0, 4096).astype(np.float64)
    _, vecs = transform.ordered_basis(W.covariance(wl, "V", 40))
    P = transform.folded_basis(vecs, 128, W.hadamard_signs(wl, "V", 40, 128))
    d = []
    for b in range(2, 9):
        rec = codec.encode_tokens(x, P, b)
        d.append(((x - codec.decode_records(rec, 128, b) @ P.T) ** 2).sum() / (x ** 2).sum())
    for b, (d0, d1) in enumerate(zip(d[:-1], d[1:]), start=2):
        hi = 4.0 * (((1 << (b + 1)) - 1) / (2.0 * ((1 << b) - 1))) ** 2
        assert 4.0 * 0.97 < d0 / d1 < hi * 1.03, (b, d0 / d1, hi)


# ------------------------------------------------------------------ attention-aware key transform (NOVA-KV)
def _nova_head(seed=3):
    wl = W.llama_t128k(2.0)
    return W.query_covariance(wl, seed % 8), W.covariance(wl, "K", seed % 8)


def test_nova_transform_reproduces_the_query_moment():
    """R_K R_K^T = M_q (the defining property of the attention-preserving transform)."""
    mq, sk = _nova_head()
    _, R, E = transform.nova_key_transform(mq, sk)
    assert np.allclose(R @ R.T, mq, rtol=1e-10, atol=1e-12 * np.abs(mq).max())
    assert np.allclose(E.T @ E, np.eye(128), atol=1e-12)


def test_nova_generalized_parseval():
    """||R_K^T (k - k^)||^2 = (k - k^)^T M_q (k - k^) for arbitrary key errors: squared
    error of the coefficients is the query-weighted key error (the orientation R^T,
    not R, is what makes it hold)."""
    mq, sk = _nova_head(5)
    _, R, _ = transform.nova_key_transform(mq, sk)
    rng = np.random.default_rng(1)
    for _ in range(5):
        e = rng.standard_normal(128)
        assert np.isclose(np.sum((R.T @ e) ** 2), e @ mq @ e, rtol=1e-10)
    e = rng.standard_normal(128)
    assert not np.isclose(np.sum((R @ e) ** 2), e @ mq @ e, rtol=1e-3)


def test_nova_coefficients_are_decorrelated_and_ordered():
    """The coefficients r = R_K^T k have covariance E^T M^(1/2) S_k M^(1/2) E: diagonal,
    equal to the returned weights in decreasing order."""
    mq, sk = _nova_head(2)
    w, R, _ = transform.nova_key_transform(mq, sk)
    c = R.T @ sk @ R
    assert np.allclose(c, np.diag(w), atol=1e-10 * w.max())
    assert np.all(np.diff(w) <= 0)


@pytest.mark.parametrize("r", [16, 64, 128])
def test_nova_bases_are_biorthogonal(r):
    mq, sk = _nova_head(4)
    P, Q = transform.nova_key_bases(mq, sk, r, W.random_basis_signs(9, r))
    assert np.allclose(P.T @ Q, np.eye(r), atol=1e-10)
    if r == 128:
        assert np.allclose(Q @ P.T, np.eye(128), atol=1e-9)


def test_nova_full_rank_unquantized_is_exact_attention():
    """Full rank, keys and values carried without quantization: folding Q_K into the
    query gives exactly softmax(q K^T / sqrt(d)) V."""
    mq, sk = _nova_head(6)
    P, Q = transform.nova_key_bases(mq, sk, 128, W.random_basis_signs(2, 128))
    rng = np.random.default_rng(4)
    k = rng.standard_normal((200, 128))
    v = rng.standard_normal((200, 128))
    qv = rng.standard_normal(128)
    got = attention.attend_coords(qv, Q, k @ P, np.eye(128), v, 1 / np.sqrt(128))
    s = k @ qv / np.sqrt(128)
    p = np.exp(s - s.max())
    assert np.allclose(got, (p / p.sum()) @ v, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("r", [16, 32, 64])
def test_nova_truncation_minimises_query_weighted_error(r):
    """Low rank (no quantization): the query-weighted key error of the transform,
    E (q . (k - k^))^2 = tr(M_q (I - Q P^T) S_k (I - Q P^T)^T), equals the sum of the
    discarded weights, and no orthonormal truncation of the same rank (the key
    covariance's own eigenbasis, or the one ordered by attention-KL weights) does better."""
    mq, sk = _nova_head(7)
    w, _, _ = transform.nova_key_transform(mq, sk)
    P, Q = transform.nova_key_bases(mq, sk, r)
    A = np.eye(128) - Q @ P.T
    err = np.trace(mq @ A @ sk @ A.T)
    assert np.isclose(err, w[r:].sum(), rtol=1e-9)
    for qc in (None, mq):
        _, vec = transform.ordered_basis(sk, qc)
        B = np.eye(128) - vec[:, :r] @ vec[:, :r].T
        assert err <= np.trace(mq @ B @ sk @ B.T) * (1 + 1e-12)


def test_attention_with_a_query_basis_reconstructs_keys_through_it():
    """attend_head_records with a separate query basis equals attention over the keys
    reconstructed as Q c^ (and the values as P_V c^_V), written out directly."""
    mq, sk = _nova_head(1)
    r = 32
    P, Q = transform.nova_key_bases(mq, sk, r, W.random_basis_signs(5, r))
    Pv = transform.folded_basis(np.linalg.qr(np.random.default_rng(2).standard_normal((128, 128)))[0], 16,
                                W.random_basis_signs(6, 16))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 128))
    xv = rng.standard_normal((300, 128))
    rk = codec.encode_tokens(x, P, 4)
    rv = codec.encode_tokens(xv, Pv, 6)
    qs = rng.standard_normal((3, 128))
    got = attention.attend_head_records(qs, P, rk, r, 4, Pv, rv, 16, 6, 0.1, query_basis=Q)
    kh = codec.decode_records(rk, r, 4) @ Q.T
    vh = codec.decode_records(rv, 16, 6) @ Pv.T
    s = qs @ kh.T * 0.1
    p = np.exp(s - s.max(axis=1, keepdims=True))
    assert np.allclose(got, (p / p.sum(axis=1, keepdims=True)) @ vh, rtol=1e-10, atol=1e-12)
