"""Shared test helpers: oracle-side calibration and caches, device transfers.

Expected values always come from ``oracle`` (CPU, float64); the GPU path only
ever receives the same inputs.
"""
from __future__ import annotations

import numpy as np

import workloads as W
from oracle import allocation, codec, packing, quantizer, transform

SCALE = 1.0 / np.sqrt(128.0)


def oracle_calibrate(wl: W.Workload):
    """(alloc, bases_k, bases_v) of a workload built with the oracle's calibration."""
    alloc, bk, bv = [], [], []
    pol = wl.allocation
    dirs = []
    for h in range(wl.n_kv_heads):
        qcov = W.query_covariance(wl, h) if (pol[0] in ("c1", "c2") and pol[2] == "kl") else None
        dirs.append((transform.ordered_basis(W.covariance(wl, "K", h), qcov),
                     transform.ordered_basis(W.covariance(wl, "V", h))))
    if pol[0] == "c2":
        n, per = wl.n_kv_heads, int(round(pol[1] * wl.head_dim))
        if pol[3] == "joint":
            pairs, _ = allocation.c2([d[0][0] for d in dirs] + [d[1][0] for d in dirs], per * 2 * n, W.C1_RANKS)
            pk_, pv_ = pairs[:n], pairs[n:]
        else:
            pk_, _ = allocation.c2([d[0][0] for d in dirs], per * n, W.C1_RANKS)
            pv_, _ = allocation.c2([d[1][0] for d in dirs], per * n, W.C1_RANKS)
    for h in range(wl.n_kv_heads):
        (wk, vk), (wv, vv) = dirs[h]
        if pol[0] == "fixed":
            a = pol[1][h]
        elif pol[0] == "c2":
            a = (pk_[h][0], pk_[h][1], pv_[h][0], pv_[h][1])
        else:
            budget = int(round(pol[1] * wl.head_dim))
            rk, b_k, _ = allocation.c1(wk, budget, W.C1_RANKS)
            rv, b_v, _ = allocation.c1(wv, budget, W.C1_RANKS)
            a = (rk, b_k, rv, b_v)
        alloc.append(tuple(a))
        bk.append(transform.folded_basis(vk, a[0], W.hadamard_signs(wl, "K", h, a[0])).astype(np.float32))
        bv.append(transform.folded_basis(vv, a[2], W.hadamard_signs(wl, "V", h, a[2])).astype(np.float32))
    return alloc, bk, bv


def oracle_cache(wl, alloc, bases_k, bases_v, batch, capacity, T, kv=None, static_k=None, static_v=None):
    """Flat K and V caches (uint32) holding the oracle's records of tokens 0..T-1.

    kv: optional dict (tensor, b, h) -> token array [T, d] (defaults to the workload's tokens).
    static_k / static_v: per-head (min, step) of header-free K / V records (None: per-token headers).
    """
    rk = [a[0] for a in alloc]
    bk = [a[1] for a in alloc]
    rv = [a[2] for a in alloc]
    bv = [a[3] for a in alloc]
    fk = [static_k is not None] * len(alloc)
    fv = [static_v is not None] * len(alloc)
    ck = np.zeros(codec.region_offsets(rk, bk, batch, capacity, fk)[-1], np.uint32)
    cv = np.zeros(codec.region_offsets(rv, bv, batch, capacity, fv)[-1], np.uint32)

    def enc(x, P, b, st):
        return codec.encode_tokens(x, P, b) if st is None else codec.encode_tokens_static(x, P, b, *st)

    for h in range(len(alloc)):
        for b in range(batch):
            xk = kv[("K", b, h)] if kv else W.tokens(wl, "K", b, h, 0, T)
            xv = kv[("V", b, h)] if kv else W.tokens(wl, "V", b, h, 0, T)
            s0, s1, _ = codec.record_slice(rk, bk, batch, capacity, h, b, 0, T, fk)
            ck[s0:s1] = enc(xk, bases_k[h], bk[h], None if static_k is None else static_k[h]).reshape(-1)
            s0, s1, _ = codec.record_slice(rv, bv, batch, capacity, h, b, 0, T, fv)
            cv[s0:s1] = enc(xv, bases_v[h], bv[h], None if static_v is None else static_v[h]).reshape(-1)
    return ck, cv


def oracle_static_scales(covs, bases, bits):
    """Each head's fixed (min, step) for header-free records: the oracle's static_scale of
    the retained coordinates' common standard deviation sqrt(trace(P^T Sigma P) / r)."""
    out = []
    for cov, P, b in zip(covs, bases, bits):
        P = np.asarray(P, np.float64)
        s = float(np.sqrt(np.trace(P.T @ np.asarray(cov, np.float64) @ P) / P.shape[1]))
        out.append(quantizer.static_scale(s, b))
    return out


def scale_words(static):
    """(min, step) pairs -> the layout's 32-bit words (fp16 min | fp16 step << 16)."""
    return [int(quantizer.fp16_bits(mu)) | (int(quantizer.fp16_bits(sg)) << 16) for mu, sg in static]


# A code may differ from the oracle's only where the two float64 projections (the
# encoder's fixed summation order, numpy's matrix product) straddle a rounding
# boundary.  Each sum of 128 products is within gamma_128 * S_j of the exact value
# (gamma_n = n u / (1 - n u), u = 2^-53, S_j = sum_i |x_i P_ij|), so the two differ
# by at most 2^-44 S_j; the subtraction and division of the code argument add a
# few ulps.  TIE_SUM_BOUND is twice that coordinate bound.
TIE_SUM_BOUND = 2.0 ** -43
TIE_FRACTION = 1e-5   # codes allowed to differ (by one, each a classified tie)


def classify_ties(x, P, r_mu, r_sg, g_c, r_c, what):
    """Every differing code must be off by one at a rounding tie: the oracle's float64
    argument (c - min) / step lies within the summation bound of the half-way point
    between the two codes.  Returns the number of differing codes."""
    tok, j = np.nonzero(g_c != r_c)
    if len(tok) == 0:
        return 0
    assert x is not None and P is not None, f"{what}: {len(tok)} codes differ and no inputs to classify them"
    x = np.asarray(x, np.float64)
    P = np.asarray(P, np.float64)
    for t, jj in zip(tok, j):
        gc, rc = int(g_c[t, jj]), int(r_c[t, jj])
        assert abs(gc - rc) == 1, f"{what}: token {t} coordinate {jj}: code {gc} against {rc}"
        c = float(x[t] @ P[:, jj])
        s_j = float(np.abs(x[t] * P[:, jj]).sum())
        mu, sg = float(r_mu[t]), float(r_sg[t])
        arg = (c - mu) / sg
        half = min(gc, rc) + 0.5
        bound = (TIE_SUM_BOUND * s_j + 2.0 ** -50 * abs(c - mu)) / sg + 2.0 ** -50 * half
        assert abs(arg - half) <= bound, (
            f"{what}: token {t} coordinate {jj}: code {gc} against {rc}, argument {arg!r} is "
            f"{abs(arg - half):.3e} from the tie at {half} (bound {bound:.3e}): not a rounding tie")
    return len(tok)


def compare_records(got, ref, r, b, what, x=None, P=None):
    """Headers exact; every differing code a classified rounding tie (off by one, the
    oracle's argument within the float64 summation bound of the half-way point), and
    at most TIE_FRACTION of the codes.  x: the tokens [n, d] the records encode, P:
    the basis [d, r] (needed only when some code differs)."""
    g_mu, g_sg, g_c = packing.unpack(got, r, b)
    r_mu, r_sg, r_c = packing.unpack(ref, r, b)
    hdr_bad = int(((g_mu != r_mu) | (g_sg != r_sg)).sum())
    assert hdr_bad == 0, f"{what}: {hdr_bad} headers differ"
    n_diff = classify_ties(x, P, r_mu, r_sg, g_c, r_c, what)
    frac = n_diff / g_c.size if g_c.size else 0.0
    assert frac <= TIE_FRACTION, f"{what}: {frac:.2e} of codes differ"
    return frac


def compare_static_records(got, ref, r, b, mu, sg, what, x=None, P=None):
    """Header-free records: every differing code a classified rounding tie (as in
    compare_records, with the head's fixed min and step), at most TIE_FRACTION of them."""
    g_c = packing.unpack_codes(got, r, b)
    r_c = packing.unpack_codes(ref, r, b)
    n = len(g_c)
    n_diff = classify_ties(x, P, np.full(n, mu), np.full(n, sg), g_c, r_c, what)
    frac = n_diff / g_c.size if g_c.size else 0.0
    assert frac <= TIE_FRACTION, f"{what}: {frac:.2e} of codes differ"
    return frac


def rel_err_per_head(got, ref):
    """max over (b, q-head) of ||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / np.maximum(den, 1e-300)).max())


# ---------------------------------------------------------------- device helpers (torch only as plumbing)
def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def u32_dev(a):
    """uint32 numpy array -> int32 device tensor with the same bits."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()


def u32_host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint32)


def oracle_calibrate_nova(wl: W.Workload):
    """(alloc, P_K list, Q_K list, P_V list) of a workload with the attention-aware key
    transform, built with the oracle: C1 on the transform's coefficient variances for the
    keys, on the value covariance's eigenvalues for the values; float32 bases."""
    budget = int(round(wl.allocation[1] * wl.head_dim))
    alloc, pk, qk, pv = [], [], [], []
    for h in range(wl.n_kv_heads):
        mq, sk = W.query_covariance(wl, h), W.covariance(wl, "K", h)
        w, _, _ = transform.nova_key_transform(mq, sk)
        rk, b_k, _ = allocation.c1(w, budget, W.C1_RANKS)
        wv, vv = transform.ordered_basis(W.covariance(wl, "V", h))
        rv, b_v, _ = allocation.c1(wv, budget, W.C1_RANKS)
        P, Q = transform.nova_key_bases(mq, sk, rk, W.hadamard_signs(wl, "K", h, rk))
        alloc.append((rk, b_k, rv, b_v))
        pk.append(P.astype(np.float32))
        qk.append(Q.astype(np.float32))
        pv.append(transform.folded_basis(vv, rv, W.hadamard_signs(wl, "V", h, rv)).astype(np.float32))
    return alloc, pk, qk, pv


def key_pairs(pk, qk):
    """The library's key basis array for a query_basis_k layout: per head P_K then Q_K."""
    return codec.concat_bases([m for pair in zip(pk, qk) for m in pair])


def to_pool(cache, ranks, bits, batch, capacity, page, pool_pages, table, fill=0xA5A5A5A5, static=None):
    """The paged form of a contiguous cache: head h's pool holds, at pool page table[b][p],
    the records of logical page p of sequence b; pool pages no entry names hold `fill`.
    Entries outside [0, pool_pages) are skipped."""
    cache = np.asarray(cache, np.uint32)
    flags = static if static is not None else [False] * len(ranks)
    src = codec.region_offsets(ranks, bits, batch, capacity, flags)
    widths = [codec.width(r, b, f) for r, b, f in zip(ranks, bits, flags)]
    dst = np.concatenate([[0], np.cumsum([pool_pages * page * w for w in widths])]).astype(np.int64)
    pool = np.full(dst[-1], fill, np.uint32)
    for h, w in enumerate(widths):
        for b in range(batch):
            for p in range(capacity // page):
                P = int(table[b][p])
                if not 0 <= P < pool_pages:
                    continue
                s0 = src[h] + (b * capacity + p * page) * w
                d0 = dst[h] + P * page * w
                pool[d0:d0 + page * w] = cache[s0:s0 + page * w]
    return pool


def from_pool(pool, ranks, bits, batch, capacity, page, pool_pages, table, fill=0, static=None):
    """The contiguous form of a paged cache (pages an entry does not name: `fill`)."""
    pool = np.asarray(pool, np.uint32)
    flags = static if static is not None else [False] * len(ranks)
    widths = [codec.width(r, b, f) for r, b, f in zip(ranks, bits, flags)]
    src = np.concatenate([[0], np.cumsum([pool_pages * page * w for w in widths])]).astype(np.int64)
    dst = codec.region_offsets(ranks, bits, batch, capacity, flags)
    out = np.full(dst[-1], fill, np.uint32)
    for h, w in enumerate(widths):
        for b in range(batch):
            for p in range(capacity // page):
                P = int(table[b][p])
                if not 0 <= P < pool_pages:
                    continue
                d0 = dst[h] + (b * capacity + p * page) * w
                s0 = src[h] + P * page * w
                out[d0:d0 + page * w] = pool[s0:s0 + page * w]
    return out


def block_table(seed, batch, pages_per_seq, pool_pages):
    """A seeded block table: distinct pool pages for every (sequence, logical page)."""
    rng = np.random.default_rng(seed)
    return rng.permutation(pool_pages)[: batch * pages_per_seq].reshape(batch, pages_per_seq).astype(np.int32)


# ---------------------------------------------------------------- vector-quantized pairs
def oracle_calibrate_nova_vq(wl: W.Workload, heads=None):
    """(alloc, P_K list, Q_K list, P_V list, K codebooks, V codebooks) of a workload with
    the attention-aware key transform at full rank and vector-quantized pairs, built
    with the oracle: columns in pair order of the coefficient variances, per-pair
    codebooks from k-means on the training sequence's tokens (float32 bases, codebooks
    [r/2, 2^b, 2] of fp16 values)."""
    from oracle import transform as T
    from oracle import vq

    bits = wl.allocation[1]
    hs = range(wl.n_kv_heads) if heads is None else heads
    alloc, pk, qk, pv, cbk, cbv = [], [], [], [], [], []
    for h in hs:
        mq, sk, sv = W.query_covariance(wl, h), W.covariance(wl, "K", h), W.covariance(wl, "V", h)
        lam_k, _, _ = T.nova_key_transform(mq, sk)
        p, q = T.nova_key_bases(mq, sk, wl.head_dim)
        ok = vq.snake_partition(lam_k)
        p, q = p[:, ok].astype(np.float32), q[:, ok].astype(np.float32)
        lam_v, ev = T.eigenbasis(sv)
        ov = vq.snake_partition(lam_v)
        v = ev[:, ov].astype(np.float32)
        xk = W.tokens(wl, "K", W.VQ_TRAIN_SEQ, h, 0, W.VQ_TRAIN_TOKENS).astype(np.float64)
        xv = W.tokens(wl, "V", W.VQ_TRAIN_SEQ, h, 0, W.VQ_TRAIN_TOKENS).astype(np.float64)
        m = wl.head_dim // 2
        cbk.append(vq.train_codebooks(xk @ p.astype(np.float64), bits, W.vq_starts(wl, "K", h, m, 1 << bits),
                                      W.VQ_ITERS))
        cbv.append(vq.train_codebooks(xv @ v.astype(np.float64), bits, W.vq_starts(wl, "V", h, m, 1 << bits),
                                      W.VQ_ITERS))
        alloc.append((wl.head_dim, bits, wl.head_dim, bits))
        pk.append(p)
        qk.append(q)
        pv.append(v)
    return alloc, pk, qk, pv, cbk, cbv


def codebook_u32(codebooks):
    """Per-head codebooks [r/2, 2^b, 2] (fp16 values) -> the library's uint32 words, heads
    concatenated (fp16 of the even coordinate low, of the odd one high)."""
    out = []
    for cb in codebooks:
        h16 = np.asarray(cb, np.float64).astype(np.float16).view(np.uint16).astype(np.uint32)
        out.append((h16[..., 0] | (h16[..., 1] << 16)).reshape(-1))
    return np.concatenate(out).astype(np.uint32)


def random_codebooks(seed, ranks, bits, scale=1.0):
    """Seeded random fp16 codebooks [r/2, 2^b, 2] per head (for format-level tests)."""
    from oracle.quantizer import fp16_round
    rng = np.random.default_rng(seed)
    return [fp16_round(rng.standard_normal((r // 2, 1 << b, 2)) * scale) for r, b in zip(ranks, bits)]


VQ_DIST_TIE = 1e-9    # distances of two codewords this close (relative) are a tie of summation order
VQ_RHO_TIE = 1e-12    # relative distance of the exact RMS from an fp16 rounding midpoint


def _fp16_midpoint_near(v, rel):
    """True where v (float64) lies within rel * |v| of a midpoint between two fp16 values."""
    v = np.asarray(v, np.float64)
    lo = np.asarray(v, np.float16).astype(np.float64)
    nxt = np.nextafter(np.asarray(lo, np.float16), np.float16(np.inf)).astype(np.float64)
    prv = np.nextafter(np.asarray(lo, np.float16), np.float16(-np.inf)).astype(np.float64)
    mids = np.stack([(lo + nxt) / 2, (lo + prv) / 2])
    return (np.abs(mids - v[None]) <= rel * np.abs(v)[None]).any(axis=0)


def compare_vq_records(got, ref, x, P, r, bits, cb, what):
    """Vector-quantized records against the oracle's: every scale word equal unless the
    oracle's exact RMS sits at an fp16 rounding midpoint (then the token is a tie), and
    every index equal unless the oracle's float64 distances to both codewords agree to
    VQ_DIST_TIE (a summation-order tie).  Returns the number of classified ties; at most
    1e-5 of the indices may be ties."""
    from oracle import vq
    got = np.asarray(got, np.uint32)
    ref = np.asarray(ref, np.uint32)
    assert got.shape == ref.shape, what
    bad = np.flatnonzero((got != ref).any(axis=1))
    if len(bad) == 0:
        return 0
    c = np.asarray(x, np.float64)[bad] @ np.asarray(P, np.float64)
    rho_exact = np.sqrt((c * c).mean(axis=1))
    rg, ig = vq.unpack_records(got[bad], r, bits)
    rr, ir = vq.unpack_records(ref[bad], r, bits)
    ties = 0
    for k, t in enumerate(bad):
        if rg[k] != rr[k]:
            assert _fp16_midpoint_near(rho_exact[k], VQ_RHO_TIE), f"{what}: token {t} scale {rg[k]} against {rr[k]}"
            ties += 1
            continue
        u = c[k] / rr[k] if rr[k] > 0 else np.zeros(r)
        for j in np.flatnonzero(ig[k] != ir[k]):
            pair = u[2 * j:2 * j + 2]
            dg = float(((pair - cb[j][ig[k, j]]) ** 2).sum())
            dr = float(((pair - cb[j][ir[k, j]]) ** 2).sum())
            assert abs(dg - dr) <= VQ_DIST_TIE * max(dr, 1e-300), \
                f"{what}: token {t} pair {j}: index {ig[k, j]} (distance {dg}) against {ir[k, j]} ({dr})"
            ties += 1
    assert ties <= max(1, 1e-5 * ref.shape[0] * (r // 2)), f"{what}: {ties} ties"
    return ties
