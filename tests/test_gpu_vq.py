"""Vector-quantized coordinate pairs (the fixed-width codebook records of the NOVA-KV
pages) on the GPU against the oracle:

* encode (prefill and append): scale words and pair indices equal to the oracle's
  except at classified float64 summation-order ties;
* decode attention over oracle-built caches, every compiled format, GQA groups 4 and
  7, ragged tails, several split sizes, through the attention-aware query basis;
  max relative error 2e-3 per (sequence, query head);
* the fused append + attend step bit-identical to append then attend;
* kv_decode reconstruction;
* the 2 bits/dim layer calibrated by the oracle (transform, pair grouping, k-means
  codebooks) end to end.
"""
import numpy as np
import pytest

import harness as H
import workloads as W
from oracle import transform, vq

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

REL_TOL = 2e-3


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_04_amd as K
    K.kv_record_words(16, 2)
    return K


def say(*a):
    print(*a, flush=True)


def _orth(seed, r):
    rng = np.random.default_rng(seed)
    return np.linalg.qr(rng.standard_normal((128, 128)))[0][:, :r].astype(np.float32)


def _vq_cache(x, bases, alloc_r, alloc_b, cbs, batch, cap, T):
    """Flat cache of the oracle's vector-quantized records of tokens 0..T-1; x[(b, h)] [T, d]."""
    widths = [vq.record_words(r, b) for r, b in zip(alloc_r, alloc_b)]
    off = np.concatenate([[0], np.cumsum([batch * cap * w for w in widths])]).astype(np.int64)
    cache = np.zeros(off[-1], np.uint32)
    for h, w in enumerate(widths):
        for b in range(batch):
            s0 = off[h] + b * cap * w
            cache[s0:s0 + T * w] = vq.encode_tokens(x[b, h], bases[h], cbs[h], alloc_b[h]).reshape(-1)
    return cache, off, widths


def _layout(K, alloc, g, B, cap, cbk, cbv, query_basis=False):
    return K.Layout(len(alloc), len(alloc) * g, B, cap, alloc, query_basis_k=query_basis,
                    codebook_k=None if cbk is None else H.u32_dev(H.codebook_u32(cbk)),
                    codebook_v=None if cbv is None else H.u32_dev(H.codebook_u32(cbv)))


def _tokens(seed, B, hkv, T, dtype=np.float16):
    rng = np.random.default_rng(seed)
    scale = np.linspace(3.0, 0.05, 128)  # unequal coordinate variances, as after a transform
    return (rng.standard_normal((B, hkv, T, 128)) * scale).astype(dtype)


# ------------------------------------------------------------------ encode
@pytest.mark.parametrize("alloc,dtype", [
    ([(128, 4, 128, 4), (64, 4, 64, 4)], "f16"),
    ([(32, 4, 32, 4), (128, 2, 128, 6)], "f32"),
])
def test_vq_encode_matches_oracle(K, alloc, dtype):
    """Prefill from an unaligned position plus one appended token; records outside the
    written range stay untouched."""
    say(f"vq encode {alloc} {dtype}")
    B, hkv, pos0, n = 2, len(alloc), 37, 700
    cap = pos0 + n + 1
    rk, bk, rv, bv = zip(*alloc)
    pk = [_orth(10 + h, r) for h, r in enumerate(rk)]
    pv = [_orth(20 + h, r) for h, r in enumerate(rv)]
    cbk = H.random_codebooks(1, rk, bk)
    cbv = H.random_codebooks(2, rv, bv)
    lay = _layout(K, alloc, 1, B, cap, cbk, cbv)
    npdt = np.float32 if dtype == "f32" else np.float16
    xk, xv = _tokens(3, B, hkv, n + 1, npdt), _tokens(4, B, hkv, n + 1, npdt)
    sentinel = 0xA5A5A5A5
    ck = H.u32_dev(np.full(K.kv_cache_bytes(lay, 0) // 4, sentinel, np.uint32))
    cv = H.u32_dev(np.full(K.kv_cache_bytes(lay, 1) // 4, sentinel, np.uint32))
    from oracle import codec
    basis_k, basis_v = H.dev(codec.concat_bases(pk)), H.dev(codec.concat_bases(pv))
    K.kv_encode(lay, H.dev(xk[:, :, :n]), H.dev(xv[:, :, :n]), n, pos0, basis_k, basis_v, ck, cv)
    K.kv_append(lay, H.dev(xk[:, :, n]), H.dev(xv[:, :, n]), pos0 + n, basis_k, basis_v, ck, cv)
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    ties = 0
    for got, ranks, bits, bases, cbs, x in ((gk, rk, bk, pk, cbk, xk), (gv, rv, bv, pv, cbv, xv)):
        widths = [vq.record_words(r, b) for r, b in zip(ranks, bits)]
        off = np.concatenate([[0], np.cumsum([B * cap * w for w in widths])]).astype(np.int64)
        for h, w in enumerate(widths):
            for b in range(B):
                s0 = off[h] + b * cap * w
                recs = got[s0:s0 + cap * w].reshape(cap, w)
                assert np.all(recs[:pos0] == sentinel), "written before pos0"
                xs = x[b, h].astype(np.float64)
                ref = vq.encode_tokens(xs, bases[h], cbs[h], bits[h])
                ties += H.compare_vq_records(recs[pos0:], ref, xs, bases[h], ranks[h], bits[h], cbs[h],
                                             f"h{h} b{b}")
    say(f"  records match ({ties} classified ties)")


def _edge_tokens(B, hkv, n, seed, dtype):
    """Zero tokens (scale 0: every coefficient normalises to 0), constant tokens,
    one non-zero dimension, repeated tokens and tokens of norm 60000, in turn."""
    rng = np.random.default_rng(seed)
    x = np.zeros((B, hkv, n, 128))
    for i in range(n):
        kind = i % 5
        if kind == 1:
            x[:, :, i] = 0.5 * (1 + i % 4)
        elif kind == 2:
            x[:, :, i, (5 * i) % 128] = 700.0 * (-1) ** i
        elif kind == 3:
            x[:, :, i] = np.linspace(-2.0, 2.0, 128)
        elif kind == 4:
            z = rng.standard_normal((B, hkv, 128))
            x[:, :, i] = z * (60000.0 / np.linalg.norm(z, axis=-1, keepdims=True))
    return x.astype(dtype)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_vq_encode_edge_tokens(K, dtype):
    """Vector-quantized records of zero, constant, one-hot, repeated and near-limit
    tokens against the oracle (prefill, then one append)."""
    say(f"vq encode edge tokens {dtype}")
    alloc = [(128, 4, 128, 4), (64, 4, 32, 6)]
    B, hkv, n = 2, len(alloc), 150
    cap = n + 1
    rk, bk, rv, bv = zip(*alloc)
    pk = [_orth(30 + h, r) for h, r in enumerate(rk)]
    pv = [_orth(40 + h, r) for h, r in enumerate(rv)]
    cbk = H.random_codebooks(5, rk, bk)
    cbv = H.random_codebooks(6, rv, bv)
    lay = _layout(K, alloc, 1, B, cap, cbk, cbv)
    npdt = np.float32 if dtype == "f32" else np.float16
    xk, xv = _edge_tokens(B, hkv, n + 1, 7, npdt), _edge_tokens(B, hkv, n + 1, 8, npdt)
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    from oracle import codec
    basis_k, basis_v = H.dev(codec.concat_bases(pk)), H.dev(codec.concat_bases(pv))
    K.kv_encode(lay, H.dev(xk[:, :, :n]), H.dev(xv[:, :, :n]), n, 0, basis_k, basis_v, ck, cv)
    K.kv_append(lay, H.dev(xk[:, :, n]), H.dev(xv[:, :, n]), n, basis_k, basis_v, ck, cv)
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    ties = 0
    for got, ranks, bits, bases, cbs, x in ((gk, rk, bk, pk, cbk, xk), (gv, rv, bv, pv, cbv, xv)):
        widths = [vq.record_words(r, b) for r, b in zip(ranks, bits)]
        off = np.concatenate([[0], np.cumsum([B * cap * w for w in widths])]).astype(np.int64)
        for h, w in enumerate(widths):
            for b in range(B):
                s0 = off[h] + b * cap * w
                recs = got[s0:s0 + cap * w].reshape(cap, w)
                xs = x[b, h].astype(np.float64)
                ref = vq.encode_tokens(xs, bases[h], cbs[h], bits[h])
                ties += H.compare_vq_records(recs, ref, xs, bases[h], ranks[h], bits[h], cbs[h], f"h{h} b{b}")
    say(f"  records match ({ties} classified ties)")


# ------------------------------------------------------------------ attention
VQ_CASES = [
    # allocation, g, batch, tokens, split
    pytest.param([(128, 4, 128, 4), (128, 4, 128, 4)], 4, 2, 3000, 0, id="r128b4-g4"),
    pytest.param([(128, 2, 128, 2), (128, 2, 128, 2)], 4, 1, 2049, 512, id="r128b2-split512"),
    pytest.param([(128, 6, 128, 6)], 4, 2, 1000, 256, id="r128b6"),
    pytest.param([(64, 4, 64, 4), (64, 4, 64, 4)], 7, 1, 1500, 0, id="r64b4-g7"),
    pytest.param([(32, 4, 32, 4)], 8, 2, 777, 256, id="r32b4-g8"),
    pytest.param([(128, 4, 64, 4), (128, 4, 64, 4)], 2, 1, 65, 0, id="r128-r64-g2"),
]


@pytest.mark.parametrize("alloc,g,B,T,split", VQ_CASES)
def test_vq_attention_matches_oracle(K, alloc, g, B, T, split):
    say(f"vq attention {alloc} g={g} B={B} T={T} split={split}")
    hkv = len(alloc)
    rk, bk, rv, bv = zip(*alloc)
    pk = [_orth(30 + h, r) for h, r in enumerate(rk)]
    pv = [_orth(40 + h, r) for h, r in enumerate(rv)]
    cbk = H.random_codebooks(5, rk, bk)
    cbv = H.random_codebooks(6, rv, bv)
    cap = T + 3
    xk, xv = _tokens(7, B, hkv, T, np.float64), _tokens(8, B, hkv, T, np.float64)
    ck, _, _ = _vq_cache(xk, pk, rk, bk, cbk, B, cap, T)
    cv, _, _ = _vq_cache(xv, pv, rv, bv, cbv, B, cap, T)
    q = W.random_vectors(9, (B, hkv * g, 128)).astype(np.float16)
    lay = _layout(K, alloc, g, B, cap, cbk, cbv)
    assert K.kv_attend_plan(lay, T)[0] == 6
    from oracle import codec
    ws = torch.zeros(K.kv_workspace_bytes(lay, T, split) // 4, dtype=torch.float32, device="cuda")
    out = torch.full((B, hkv * g, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q), T, H.dev(codec.concat_bases(pk)), H.dev(codec.concat_bases(pv)),
                       H.u32_dev(ck), H.u32_dev(cv), H.SCALE, out, ws, split_tokens=split)
    torch.cuda.synchronize()
    ref = vq.attend_cache(q.astype(np.float64), pk, pv, ck, cv, alloc, B, cap, T, H.SCALE, cbk, cbv)
    err = H.rel_err_per_head(out.cpu().numpy(), ref)
    say(f"  max rel err {err:.3e}")
    assert err <= REL_TOL


def test_vq_keys_with_scalar_values(K):
    """Only the keys vector-quantized: the value records keep the scalar format."""
    from oracle import codec
    alloc = [(128, 4, 128, 2), (64, 4, 64, 4)]
    hkv, g, B, T = 2, 4, 1, 1200
    rk, bk, rv, bv = zip(*alloc)
    pk = [_orth(50 + h, r) for h, r in enumerate(rk)]
    pv = [_orth(60 + h, r) for h, r in enumerate(rv)]
    cbk = H.random_codebooks(7, rk, bk)
    xk, xv = _tokens(11, B, hkv, T, np.float64), _tokens(12, B, hkv, T, np.float64)
    ck, _, _ = _vq_cache(xk, pk, rk, bk, cbk, B, T, T)
    cv = H.oracle_cache(W.LLAMA_T32K, alloc, pk, pv, B, T, T,
                        kv={(t, b, h): (xk if t == "K" else xv)[b, h] for t in "KV" for b in range(B)
                            for h in range(hkv)})[1]
    lay = _layout(K, alloc, g, B, T, cbk, None)
    assert K.kv_attend_plan(lay, T)[0] == 6
    q = W.random_vectors(13, (B, hkv * g, 128)).astype(np.float16)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q), T, H.dev(codec.concat_bases(pk)), H.dev(codec.concat_bases(pv)),
                       H.u32_dev(ck), H.u32_dev(cv), H.SCALE, out, ws)
    torch.cuda.synchronize()
    ref = vq.attend_cache(q.astype(np.float64), pk, pv, ck, cv, alloc, B, T, T, H.SCALE, cbk, None)
    assert H.rel_err_per_head(out.cpu().numpy(), ref) <= REL_TOL


def test_vq_fused_step_and_decode(K):
    """kv_append_attend_decode equals kv_append + kv_attend_decode bit for bit, the
    appended records are the oracle's, and kv_decode reconstructs rho * codeword."""
    from oracle import codec
    alloc = [(128, 4, 128, 4), (64, 4, 64, 4)]
    hkv, g, B, T = 2, 4, 2, 1800
    rk, bk, rv, bv = zip(*alloc)
    pk = [_orth(70 + h, r) for h, r in enumerate(rk)]
    pv = [_orth(80 + h, r) for h, r in enumerate(rv)]
    cbk, cbv = H.random_codebooks(9, rk, bk), H.random_codebooks(10, rv, bv)
    xk, xv = _tokens(14, B, hkv, T, np.float16), _tokens(15, B, hkv, T, np.float16)
    ck_h, _, _ = _vq_cache(xk[:, :, :T - 1].astype(np.float64), pk, rk, bk, cbk, B, T, T - 1)
    cv_h, _, _ = _vq_cache(xv[:, :, :T - 1].astype(np.float64), pv, rv, bv, cbv, B, T, T - 1)
    lay = _layout(K, alloc, g, B, T, cbk, cbv)
    basis_k, basis_v = H.dev(codec.concat_bases(pk)), H.dev(codec.concat_bases(pv))
    q = H.dev(W.random_vectors(16, (B, hkv * g, 128)).astype(np.float16))
    k1, v1 = H.dev(xk[:, :, T - 1]), H.dev(xv[:, :, T - 1])
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    ck_f, cv_f = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_f = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    K.kv_append_attend_decode(lay, k1, v1, q, T, basis_k, basis_v, ck_f, cv_f, H.SCALE, out_f, ws)
    ck_s, cv_s = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_s = torch.empty_like(out_f)
    K.kv_append(lay, k1, v1, T - 1, basis_k, basis_v, ck_s, cv_s)
    K.kv_attend_decode(lay, q, T, basis_k, basis_v, ck_s, cv_s, H.SCALE, out_s, ws)
    torch.cuda.synchronize()
    assert torch.equal(ck_f, ck_s) and torch.equal(cv_f, cv_s)
    assert torch.equal(out_f, out_s)
    gk, gv = H.u32_host(ck_f), H.u32_host(cv_f)
    for got, ranks, bits, bases, cbs, x in ((gk, rk, bk, pk, cbk, xk), (gv, rv, bv, pv, cbv, xv)):
        widths = [vq.record_words(r, b) for r, b in zip(ranks, bits)]
        off = np.concatenate([[0], np.cumsum([B * T * w for w in widths])]).astype(np.int64)
        for h, w in enumerate(widths):
            for b in range(B):
                s0 = off[h] + (b * T + T - 1) * w
                xs = x[b, h, T - 1:T].astype(np.float64)
                H.compare_vq_records(got[s0:s0 + w][None], vq.encode_tokens(xs, bases[h], cbs[h], bits[h]), xs,
                                     bases[h], ranks[h], bits[h], cbs[h], f"appended h{h} b{b}")
    ref = vq.attend_cache(q.cpu().numpy().astype(np.float64), pk, pv, gk, gv, alloc, B, T, T, H.SCALE, cbk, cbv)
    assert H.rel_err_per_head(out_f.cpu().numpy(), ref) <= REL_TOL
    # reconstruction
    for which, cache, bases, ranks, bits, cbs in ((0, ck_f, basis_k, rk, bk, cbk), (1, cv_f, basis_v, rv, bv, cbv)):
        o = torch.empty((B, hkv, T, 128), dtype=torch.float32, device="cuda")
        K.kv_decode(lay, which, T, 0, bases, cache, o)
        torch.cuda.synchronize()
        host = H.u32_host(cache)
        widths = [vq.record_words(r, b) for r, b in zip(ranks, bits)]
        off = np.concatenate([[0], np.cumsum([B * T * w for w in widths])]).astype(np.int64)
        P = pk if which == 0 else pv
        for h, w in enumerate(widths):
            for b in range(B):
                s0 = off[h] + b * T * w
                c = vq.decode_records(host[s0:s0 + T * w].reshape(T, w), ranks[h], bits[h], cbs[h])
                ref = c @ P[h].astype(np.float64).T
                bound = (ranks[h] + 2) * 2.0 ** -24 * (np.abs(c) @ np.abs(P[h].astype(np.float64)).T) + 1e-30
                assert np.all(np.abs(o[b, h].cpu().numpy() - ref) <= bound)


def test_vq_calibrated_layer_end_to_end(K):
    """Two KV heads of the 128K LLaMA-shaped layer at 2 bits per coordinate, calibrated
    by the oracle: attention-aware key transform, pair grouping and k-means codebooks.
    GPU encode then attend against the oracle's encode then attend."""
    from oracle import codec
    wl = W.llama_t128k_nova_vq(2.0)
    alloc, pk, qk, pv, cbk, cbv = H.oracle_calibrate_nova_vq(wl, heads=[0, 1])
    B, T, g = 1, 2500, wl.group
    hkv = len(alloc)
    xk = np.stack([np.stack([W.tokens(wl, "K", b, h, 0, T) for h in range(hkv)]) for b in range(B)])
    xv = np.stack([np.stack([W.tokens(wl, "V", b, h, 0, T) for h in range(hkv)]) for b in range(B)])
    lay = _layout(K, alloc, g, B, T, cbk, cbv, query_basis=True)
    kb = H.dev(np.concatenate([np.concatenate([p.reshape(-1), q.reshape(-1)]) for p, q in zip(pk, qk)]))
    vb = H.dev(codec.concat_bases(pv))
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    K.kv_encode(lay, H.dev(xk), H.dev(xv), T, 0, kb, vb, ck, cv)
    q = W.query_array(wl)[:B, :hkv * g]
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q), T, kb, vb, ck, cv, H.SCALE, out, ws)
    torch.cuda.synchronize()
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bk, rv, bv = zip(*alloc)
    ok_, _, wk = _vq_cache(xk.astype(np.float64), pk, rk, bk, cbk, B, T, T)
    ov_, _, _ = _vq_cache(xv.astype(np.float64), pv, rv, bv, cbv, B, T, T)
    ties = 0
    for got, ref, ranks, bits, bases, cbs, x in ((gk, ok_, rk, bk, pk, cbk, xk), (gv, ov_, rv, bv, pv, cbv, xv)):
        w = vq.record_words(ranks[0], bits[0])
        for h in range(hkv):
            for b in range(B):
                s0 = (h * B + b) * T * w
                ties += H.compare_vq_records(got[s0:s0 + T * w].reshape(T, w), ref[s0:s0 + T * w].reshape(T, w),
                                             x[b, h].astype(np.float64), bases[h], ranks[h], bits[h], cbs[h],
                                             f"h{h} b{b}")
    ref = vq.attend_cache(np.asarray(q, np.float64), pk, pv, gk, gv, alloc, B, T, T, H.SCALE, cbk, cbv,
                          query_bases=qk)
    err = H.rel_err_per_head(out.cpu().numpy(), ref)
    say(f"calibrated 2 bits/dim layer: {ties} ties, max rel err {err:.3e}")
    assert err <= REL_TOL


def test_vq_full_size_128k_sampled_units(K):
    """The vector-quantized 128K layer at full size (4 sequences x 8 KV heads x 131073
    tokens, 2 bits per coordinate; calibrated by the oracle: attention-aware key transform,
    pair grouping, k-means codebooks), encoded on the GPU and attended with the default
    split plan, the configuration the benchmark times.  Sampled (sequence, KV head) units
    are re-encoded by the oracle from the same inputs: their records must match (classified
    ties only) and their query heads' outputs match oracle attention."""
    from oracle import codec
    wl = W.llama_t128k_nova_vq(2.0)
    T = wl.context + 1
    B, hkv, hq, d, g = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.group
    alloc, pk, qk, pv, cbk, cbv = H.oracle_calibrate_nova_vq(wl)
    say(f"full size {wl.name}")
    lay = _layout(K, alloc, g, B, T, cbk, cbv, query_basis=True)
    kb = H.dev(np.concatenate([np.concatenate([p.reshape(-1), q.reshape(-1)]) for p, q in zip(pk, qk)]))
    vb = H.dev(codec.concat_bases(pv))
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    for t0 in range(0, T, 1 << 15):
        n = min(1 << 15, T - t0)
        K.kv_encode(lay, H.dev(W.kv_array(wl, "K", t0, n)), H.dev(W.kv_array(wl, "V", t0, n)), n, t0, kb, vb, ck, cv)
    q = W.query_array(wl, 0)
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q), T, kb, vb, ck, cv, H.SCALE, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    w = vq.record_words(d, alloc[0][1])
    for b, h in [(0, 0), (B - 1, hkv - 1)]:
        xk = W.tokens(wl, "K", b, h, 0, T).astype(np.float64)
        xv = W.tokens(wl, "V", b, h, 0, T).astype(np.float64)
        rk = np.concatenate([vq.encode_tokens(xk[i:i + 16384], pk[h], cbk[h], alloc[h][1]) for i in range(0, T, 16384)])
        rv = np.concatenate([vq.encode_tokens(xv[i:i + 16384], pv[h], cbv[h], alloc[h][3]) for i in range(0, T, 16384)])
        s0 = (h * B + b) * T * w
        tk = H.compare_vq_records(gk[s0:s0 + T * w].reshape(T, w), rk, xk, pk[h], d, alloc[h][1], cbk[h], f"K b{b} h{h}")
        tv = H.compare_vq_records(gv[s0:s0 + T * w].reshape(T, w), rv, xv, pv[h], d, alloc[h][3], cbv[h], f"V b{b} h{h}")
        ck_ = vq.decode_records(rk, d, alloc[h][1], cbk[h])
        cv_ = vq.decode_records(rv, d, alloc[h][3], cbv[h])
        from oracle import attention
        ref = np.stack([attention.attend_coords(qq, qk[h], ck_, pv[h], cv_, H.SCALE)
                        for qq in q[b, h * g:(h + 1) * g].astype(np.float64)])
        err = H.rel_err_per_head(got[b, h * g:(h + 1) * g], ref)
        say(f"  unit (b={b}, h={h}): ties K {tk} V {tv}, max rel err {err:.3e}")
        assert err <= REL_TOL
