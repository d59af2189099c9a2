"""Pins of the oracle's fixed-width vector quantizer (oracle/vq.py) against what the
pages and the mathematics fix: the volume-equalising grouping on spectra whose group
volumes have a closed form, Lloyd's k-means against the textbook Lloyd-Max quantizers
of the Gaussian, the fixed point of Lloyd's iteration, hand-worked records, exact
round trips, and the generalised Parseval relation of the attention-aware key
transform through the vector quantizer."""
import numpy as np
import pytest

import workloads as W
from oracle import attention, transform, vq
from oracle.quantizer import fp16_round


# ----------------------------------------------------------------- grouping
def test_snake_partition_hand_worked():
    """Eight coefficients with variances 2^3 .. 2^-4 in decreasing order: groups
    {0, 7}, {1, 6}, {2, 5}, {3, 4}; every group's volume is 2^-1."""
    v = 2.0 ** -np.arange(-3, 5)
    perm = vq.snake_partition(v)
    assert perm.tolist() == [0, 7, 1, 6, 2, 5, 3, 4]
    assert np.allclose(vq.group_log_volumes(v, perm), np.log(0.5), atol=1e-15)


def test_snake_partition_sorts_first():
    """The deal follows the variances, not the input order."""
    v = np.array([0.25, 8.0, 1.0, 0.0625, 4.0, 0.5, 2.0, 0.125])
    perm = vq.snake_partition(v)
    assert sorted(perm.tolist()) == list(range(8))
    assert [v[i] for i in perm] == [8.0, 0.0625, 4.0, 0.125, 2.0, 0.25, 1.0, 0.5]


@pytest.mark.parametrize("r", [16, 64, 128])
def test_snake_partition_equalises_geometric_volumes(r):
    """For a geometric spectrum the back-and-forth deal gives every pair the same
    volume exactly (log volume = log(l0 * l_{r-1})), while a plain round-robin deal
    spreads the log volumes over (r - 2) * |log(ratio)|."""
    ratio = 0.93
    v = 3.0 * ratio ** np.arange(r)
    lv = vq.group_log_volumes(v, vq.snake_partition(v))
    assert np.allclose(lv, np.log(v[0] * v[-1]), rtol=0, atol=1e-12)
    rr = np.concatenate([[g, g + r // 2] for g in range(r // 2)])  # round-robin: rank g and g + r/2
    spread = np.ptp(vq.group_log_volumes(v, rr))
    assert spread == pytest.approx((r - 2) * abs(np.log(ratio)), rel=1e-9)


# ----------------------------------------------------------------- k-means
def _gauss(n, seed):
    return np.random.default_rng(seed).standard_normal(n)


@pytest.mark.parametrize("K,levels,mse", [
    (2, [-np.sqrt(2 / np.pi), np.sqrt(2 / np.pi)], 1 - 2 / np.pi),  # closed form
    (4, [-1.5104, -0.4528, 0.4528, 1.5104], 0.1175),                # Lloyd-Max (Max, 1960)
])
def test_kmeans_reaches_the_lloyd_max_gaussian_quantizer(K, levels, mse):
    """On 400k N(0, 1) samples Lloyd's algorithm converges to the optimal scalar
    quantizer of the Gaussian: centroids +-sqrt(2/pi) with MSE 1 - 2/pi for two
    levels, +-0.4528 and +-1.5104 with MSE 0.1175 for four."""
    x = _gauss(400_000, 3)[:, None]
    init = np.linspace(-1.0, 1.0, K)[:, None]
    cb, assign, hist = vq.kmeans(x, init, 200)
    assert np.allclose(np.sort(cb[:, 0]), levels, atol=0.01)
    assert hist[-1] == pytest.approx(mse, abs=0.002)


def test_kmeans_fixed_point_and_monotone_distortion():
    """Lloyd's iteration never increases the distortion, and once the assignment is
    stable every codeword is the mean of its cell and every point sits in the cell of
    a nearest codeword (checked by brute force)."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5000, 2)) * np.array([2.0, 0.5])
    cb, assign, hist = vq.kmeans(x, x[:16], 500)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))
    for e in range(16):
        cell = x[assign == e]
        if len(cell):
            assert np.allclose(cb[e], cell.mean(axis=0), rtol=0, atol=1e-12)
    d = ((x[:, None, :] - cb[None]) ** 2).sum(-1)
    assert np.allclose(d[np.arange(len(x)), assign], d.min(axis=1), rtol=0, atol=0)


def test_nearest_takes_the_first_on_ties():
    cb = np.array([[5.0, 5.0], [1.0, 0.0], [9.0, 9.0], [-1.0, 0.0]])
    assert vq.nearest(np.array([[0.0, 0.0]]), cb).tolist() == [1]
    assert vq.nearest(np.array([[-1.0, 0.0], [8.0, 8.0]]), cb).tolist() == [3, 2]


def test_train_codebooks_fp16_and_per_pair():
    """Codebooks are per pair, 2^b codewords each, stored as fp16 values; pairs whose
    training values are exactly the four points (+-1, +-1) (every token then has RMS 1)
    recover those points from starting points that hold them."""
    rng = np.random.default_rng(4)
    n = 4000
    pts = np.array([[1.0, 1.0], [-1.0, 1.0], [1.0, -1.0], [-1.0, -1.0]])
    c = np.concatenate([pts[rng.integers(0, 4, n)], pts[rng.integers(0, 4, n)]], axis=1)
    init = [np.array([int(np.flatnonzero((c[:, 2 * g:2 * g + 2] == p).all(1))[0]) for p in pts]) for g in range(2)]
    cb = vq.train_codebooks(c, 2, init, iters=10)
    assert cb.shape == (2, 4, 2)
    assert np.array_equal(cb, fp16_round(cb))
    assert np.array_equal(cb[0], pts) and np.array_equal(cb[1], pts)


# ----------------------------------------------------------------- records
def test_rms_scale_hand_worked():
    c = np.array([[3.0, 4.0], [0.0, 0.0], [1.0, 1.0]])
    rho = vq.rms_scale(c)
    # sqrt(12.5) = 3.5355339...: the fp16 neighbours are 3.533203125 and 3.53515625
    assert rho.tolist() == [3.53515625, 0.0, 1.0]
    u = vq.normalise(c, rho)
    assert np.array_equal(u[1], [0.0, 0.0]) and np.array_equal(u[2], [1.0, 1.0])


def test_record_words_hand_worked():
    """r = 4 coefficients (two pairs), 2-bit indices 1 and 3, rho = 2: word 0 =
    0x4000 << 16 (fp16 2.0 as the step, fp16 +0 as the minimum), word 1 = 1 | 3 << 2."""
    cb = np.zeros((2, 4, 2))
    cb[0, 1] = [2.0, 0.0]
    cb[1, 3] = [0.0, -2.0]
    # mean square 4 (up to one rounding), so rho = fp16(2.0...) = 2; u = (+-sqrt 2, 0)
    # is nearer to (2, 0) than to (0, 0), and likewise for the second pair
    c = np.array([[2.0, 0.0, 0.0, -2.0]]) * np.sqrt(2.0)
    words = vq.encode_coords(c, cb, 2)
    assert words.shape == (1, vq.record_words(4, 2)) == (1, 2)
    assert words[0].tolist() == [0x4000 << 16, 1 | (3 << 2)]
    rho, idx = vq.unpack_records(words, 4, 2)
    assert rho.tolist() == [2.0] and idx.tolist() == [[1, 3]]


@pytest.mark.parametrize("r,bits", [(16, 2), (32, 4), (128, 4), (64, 8)])
def test_exact_round_trip_on_codewords(r, bits):
    """Tokens built as rho * (codewords whose entries are all +-1) have RMS exactly
    rho, so they encode to those codewords and decode to themselves bit for bit."""
    rng = np.random.default_rng(r + bits)
    K = 1 << bits
    cb = rng.choice([-1.0, 1.0], size=(r // 2, K, 2))
    n = 50
    idx = rng.integers(0, K, (n, r // 2))
    rho = fp16_round(rng.uniform(0.01, 300.0, n))
    c = rho[:, None] * cb[np.arange(r // 2)[None, :], idx].reshape(n, r)
    words = vq.encode_coords(c, cb, bits)
    r2, i2 = vq.unpack_records(words, r, bits)
    # duplicated codewords may be picked earlier: the reconstruction is what is exact
    assert np.array_equal(r2, rho)
    assert np.array_equal(vq.decode_records(words, r, bits, cb), c)
    assert np.all(i2 <= idx)


def test_zero_token():
    """rho = 0: the normalised pairs are zero, each index is the codeword nearest the
    origin, and the reconstruction is zero."""
    cb = np.arange(2 * 4 * 2, dtype=np.float64).reshape(2, 4, 2) - 5.0
    words = vq.encode_coords(np.zeros((1, 4)), cb, 2)
    # pair 0 codewords (-5,-4) (-3,-2) (-1,0) (1,2): nearest to 0 is index 2; pair 1 (3,4)...: index 0
    assert words[0].tolist() == [0, 2 | (0 << 2)]
    assert np.array_equal(vq.decode_records(words, 4, 2, cb), np.zeros((1, 4)))


def test_encode_is_brute_force_nearest():
    """Every index is the brute-force nearest codeword of the normalised pair."""
    rng = np.random.default_rng(12)
    r, bits = 8, 3
    cb = fp16_round(rng.standard_normal((r // 2, 1 << bits, 2)))
    c = rng.standard_normal((200, r)) * 5
    _, idx = vq.unpack_records(vq.encode_coords(c, cb, bits), r, bits)
    rho = vq.rms_scale(c)
    for t in range(200):
        for g in range(r // 2):
            u = c[t, 2 * g:2 * g + 2] / rho[t]
            d = [float((u[0] - w[0]) ** 2 + (u[1] - w[1]) ** 2) for w in cb[g]]
            assert idx[t, g] == int(np.argmin(d))


# ----------------------------------------------------------------- with the transforms
def test_parseval_through_the_vector_quantizer():
    """With the attention-aware key transform at full rank (P_K = M^(1/2) E encodes,
    Q_K = M^(-1/2) E reconstructs), the transform-domain error of the quantized
    coefficients equals the M-weighted key error: ||c - c^||^2 = (k - k^)^T M (k - k^)."""
    wl = W.llama_t128k_nova(2.0)
    mq, sk = W.query_covariance(wl, 1), W.covariance(wl, "K", 1)
    P, Q = transform.nova_key_bases(mq, sk, 128)
    k = W.tokens(wl, "K", 0, 1, 0, 300, "f64")
    c = k @ P
    rng = np.random.default_rng(2)
    cb = fp16_round(rng.standard_normal((64, 16, 2)))
    ch = vq.decode_records(vq.encode_coords(c, cb, 4), 128, 4, cb)
    kh = ch @ Q.T
    lhs = ((c - ch) ** 2).sum(axis=1)
    rhs = np.einsum("ti,ij,tj->t", k - kh, mq, k - kh)
    assert np.allclose(lhs, rhs, rtol=1e-8)


def test_attention_over_vq_records_is_textbook_attention():
    """Attention over vector-quantized records equals softmax attention written out
    over the reconstructed keys Q_K c^_K and values P_V c^_V."""
    rng = np.random.default_rng(5)
    r, bits, T, g = 16, 3, 40, 2
    Pk = np.linalg.qr(rng.standard_normal((128, r)))[0]
    Pv = np.linalg.qr(rng.standard_normal((128, r)))[0]
    cbk = fp16_round(rng.standard_normal((r // 2, 1 << bits, 2)))
    cbv = fp16_round(rng.standard_normal((r // 2, 1 << bits, 2)))
    k = rng.standard_normal((T, 128))
    v = rng.standard_normal((T, 128))
    ck = vq.encode_tokens(k, Pk, cbk, bits).reshape(-1)
    cv = vq.encode_tokens(v, Pv, cbv, bits).reshape(-1)
    q = rng.standard_normal((1, g, 128))
    scale = 1 / np.sqrt(128)
    got = vq.attend_cache(q, [Pk], [Pv], ck, cv, [(r, bits, r, bits)], 1, T, T, scale, [cbk], [cbv])
    kh = vq.decode_records(ck.reshape(T, -1), r, bits, cbk) @ Pk.T
    vh = vq.decode_records(cv.reshape(T, -1), r, bits, cbv) @ Pv.T
    for i in range(g):
        s = kh @ q[0, i] * scale
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(got[0, i], p @ vh, rtol=1e-12, atol=1e-12)
    # a scalar value tensor mixes with vector-quantized keys through the same call
    from oracle import codec
    cv2 = codec.encode_tokens(v, Pv, 4).reshape(-1)
    got2 = vq.attend_cache(q, [Pk], [Pv], ck, cv2, [(r, bits, r, 4)], 1, T, T, scale, [cbk], None)
    vh2 = codec.decode_records(cv2.reshape(T, -1), r, 4) @ Pv.T
    s = kh @ q[0, 0] * scale
    p = attention.softmax(s)
    assert np.allclose(got2[0, 0], p @ vh2, rtol=1e-12, atol=1e-12)
