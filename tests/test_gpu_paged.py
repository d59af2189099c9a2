"""Paged caches: each head's region a pool of fixed-size pages, a block table mapping
every sequence's logical pages to pool pages.  The kernels are the contiguous ones
with another record address, so a paged call must reproduce the contiguous call bit
for bit (same splits, tiles and summation order): attention (specialised and generic
kernels, ragged lengths), prefill encode and append, the fused step, kv_decode; and
match the oracle.  Pool pages no entry names are never written; an entry outside the
pool writes nothing and reads as zeros."""
import numpy as np
import pytest

import harness as H
import workloads as W
from oracle import attention, codec, transform

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

REL_TOL = 2e-3
FILL = 0xA5A5A5A5


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_04_amd as K
    K.kv_record_words(16, 2)
    return K


def say(*a):
    print(*a, flush=True)


def _bases(alloc, seed):
    bk, bv = [], []
    for h, (rk, _, rv, _) in enumerate(alloc):
        bk.append(transform.basis_for_head(W.random_covariance(seed + h, 128), rk,
                                           W.random_basis_signs(seed + 20 + h, rk)).astype(np.float32))
        bv.append(transform.basis_for_head(W.random_covariance(seed + 40 + h, 128), rv,
                                           W.random_basis_signs(seed + 60 + h, rv)).astype(np.float32))
    return bk, bv


@pytest.mark.parametrize("alloc", [[(64, 4, 32, 8), (32, 8, 64, 4)], [(32, 3, 64, 5), (16, 7, 128, 6)]],
                         ids=["specialised", "generic"])
def test_paged_attention_equals_contiguous(K, alloc):
    wl = W.LLAMA_T32K
    B, g, cap, T, page = 3, 4, 4096, 3000, 256
    pps, pool_pages = cap // page, cap // page * B + 5
    hkv = len(alloc)
    bk, bv = _bases(alloc, 7)
    kv = {(t, b, h): W.tokens(wl, t, b, h, 0, T) for t in "KV" for b in range(B) for h in range(hkv)}
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T, kv=kv)
    table = H.block_table(3, B, pps, pool_pages)
    rk, bits_k, rv, bits_v = zip(*alloc)
    pk_h = H.to_pool(ck_h, rk, bits_k, B, cap, page, pool_pages, table)
    pv_h = H.to_pool(cv_h, rv, bits_v, B, cap, page, pool_pages, table)
    q = H.dev(W.random_vectors(9, (B, hkv * g, 128)).astype(np.float16), torch.float16)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    lay_c = K.Layout(hkv, hkv * g, B, cap, alloc)
    bt = torch.from_numpy(table).cuda()
    lay_p = K.Layout(hkv, hkv * g, B, cap, alloc, page_tokens=page, pool_pages=pool_pages, block_table=bt)
    assert K.kv_cache_bytes(lay_p, 0) == 4 * len(pk_h)
    ws = torch.zeros(K.kv_workspace_bytes(lay_c, T) // 4, dtype=torch.float32, device="cuda")
    out_c = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    out_p = torch.empty_like(out_c)
    K.kv_attend_decode(lay_c, q, T, pk, pv, H.u32_dev(ck_h), H.u32_dev(cv_h), H.SCALE, out_c, ws)
    ckp, cvp = H.u32_dev(pk_h), H.u32_dev(pv_h)
    K.kv_attend_decode(lay_p, q, T, pk, pv, ckp, cvp, H.SCALE, out_p, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p), "paged attention differs from contiguous"
    ref = attention.attend_cache(q.cpu().numpy().astype(np.float64), bk, bv, ck_h, cv_h, alloc, B, cap, T, H.SCALE)
    err = H.rel_err_per_head(out_p.cpu().numpy(), ref)
    say(f"paged attention {alloc}: bit-equal to contiguous, max rel err {err:.3e}")
    assert err <= REL_TOL
    # ragged lengths through the same pages
    lens = torch.tensor([2999, 700, 1], dtype=torch.int32, device="cuda")
    K.kv_attend_decode_ragged(lay_c, q, lens, T, pk, pv, H.u32_dev(ck_h), H.u32_dev(cv_h), H.SCALE, out_c, ws)
    K.kv_attend_decode_ragged(lay_p, q, lens, T, pk, pv, ckp, cvp, H.SCALE, out_p, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p), "paged ragged attention differs from contiguous"


def test_paged_encode_append_and_fused_step(K):
    """Prefill encode from an unaligned position across pages, then one fused decode step:
    the pool gathered back equals the contiguous cache bit for bit, unnamed pool pages
    keep their fill, and the outputs are equal."""
    wl = W.LLAMA_T32K
    alloc = [(128, 2, 64, 4), (16, 6, 32, 5)]
    B, g, cap, page = 2, 4, 2048, 128
    pos0, n = 100, 1500
    T = pos0 + n + 1
    pps, pool_pages = cap // page, cap // page * B + 3
    hkv = len(alloc)
    bk, bv = _bases(alloc, 21)
    rk, bits_k, rv, bits_v = zip(*alloc)
    table = H.block_table(5, B, pps, pool_pages)
    bt = torch.from_numpy(table).cuda()
    lay_c = K.Layout(hkv, hkv * g, B, cap, alloc)
    lay_p = K.Layout(hkv, hkv * g, B, cap, alloc, page_tokens=page, pool_pages=pool_pages, block_table=bt)
    x = {t: np.stack([np.stack([W.tokens(wl, t, b, h, 0, T) for h in range(hkv)]) for b in range(B)]) for t in "KV"}
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    ck_c = H.u32_dev(np.zeros(K.kv_cache_bytes(lay_c, 0) // 4, np.uint32))
    cv_c = H.u32_dev(np.zeros(K.kv_cache_bytes(lay_c, 1) // 4, np.uint32))
    ck_p = H.u32_dev(np.full(K.kv_cache_bytes(lay_p, 0) // 4, FILL, np.uint32))
    cv_p = H.u32_dev(np.full(K.kv_cache_bytes(lay_p, 1) // 4, FILL, np.uint32))
    for lay, ck, cv in ((lay_c, ck_c, cv_c), (lay_p, ck_p, cv_p)):
        K.kv_encode(lay, H.dev(x["K"][:, :, pos0:pos0 + n]), H.dev(x["V"][:, :, pos0:pos0 + n]), n, pos0, pk, pv, ck, cv)
    gk_c, gv_c = H.u32_host(ck_c), H.u32_host(cv_c)
    gk_p, gv_p = H.u32_host(ck_p), H.u32_host(cv_p)
    for got_c, got_p, ranks, bits in ((gk_c, gk_p, rk, bits_k), (gv_c, gv_p, rv, bits_v)):
        back = H.from_pool(got_p, ranks, bits, B, cap, page, pool_pages, table)
        for h in range(hkv):
            for b in range(B):
                s0, s1, _ = codec.record_slice(ranks, bits, B, cap, h, b, pos0, pos0 + n)
                assert np.array_equal(back[s0:s1], got_c[s0:s1]), f"head {h} sequence {b}"
        named = H.to_pool(np.zeros_like(got_c), ranks, bits, B, cap, page, pool_pages, table, fill=FILL)
        assert np.all(got_p[named == FILL] == FILL), "a pool page no entry names was written"
    q = H.dev(W.random_vectors(11, (B, hkv * g, 128)).astype(np.float16), torch.float16)
    k1 = H.dev(x["K"][:, :, T - 1])
    v1 = H.dev(x["V"][:, :, T - 1])
    ws = torch.zeros(K.kv_workspace_bytes(lay_c, T) // 4, dtype=torch.float32, device="cuda")
    out_c = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    out_p = torch.empty_like(out_c)
    K.kv_append_attend_decode(lay_c, k1, v1, q, T, pk, pv, ck_c, cv_c, H.SCALE, out_c, ws)
    K.kv_append_attend_decode(lay_p, k1, v1, q, T, pk, pv, ck_p, cv_p, H.SCALE, out_p, ws)
    torch.cuda.synchronize()
    # tokens 0 .. pos0-1 were never written: zero in the contiguous cache, fill in the pool
    # pages of the first sequence pages; compare the step only where both hold records
    assert torch.isfinite(out_c).all()
    gk_c, gk_p = H.u32_host(ck_c), H.u32_host(ck_p)
    back = H.from_pool(gk_p, rk, bits_k, B, cap, page, pool_pages, table)
    for h in range(hkv):
        for b in range(B):
            s0, s1, _ = codec.record_slice(rk, bits_k, B, cap, h, b, pos0, T)
            assert np.array_equal(back[s0:s1], gk_c[s0:s1]), "fused append record differs"
    # a fully encoded context: the same step on both layouts gives the same bits
    K.kv_encode(lay_c, H.dev(x["K"][:, :, :pos0]), H.dev(x["V"][:, :, :pos0]), pos0, 0, pk, pv, ck_c, cv_c)
    K.kv_encode(lay_p, H.dev(x["K"][:, :, :pos0]), H.dev(x["V"][:, :, :pos0]), pos0, 0, pk, pv, ck_p, cv_p)
    K.kv_attend_decode(lay_c, q, T, pk, pv, ck_c, cv_c, H.SCALE, out_c, ws)
    K.kv_attend_decode(lay_p, q, T, pk, pv, ck_p, cv_p, H.SCALE, out_p, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p)
    kc = {(t, b, h): x[t][b, h] for t in "KV" for b in range(B) for h in range(hkv)}
    ok_h, ov_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T, kv=kc)
    ref = attention.attend_cache(q.cpu().numpy().astype(np.float64), bk, bv, ok_h, ov_h, alloc, B, cap, T, H.SCALE)
    err = H.rel_err_per_head(out_p.cpu().numpy(), ref)
    say(f"paged encode + fused step: bit-equal to contiguous, max rel err {err:.3e}")
    assert err <= REL_TOL
    # kv_decode through the pages
    for which, cc, cp in ((0, ck_c, ck_p), (1, cv_c, cv_p)):
        oc = torch.empty((B, hkv, T, 128), dtype=torch.float32, device="cuda")
        op = torch.empty_like(oc)
        basis = pk if which == 0 else pv
        K.kv_decode(lay_c, which, T, 0, basis, cc, oc)
        K.kv_decode(lay_p, which, T, 0, basis, cp, op)
        torch.cuda.synchronize()
        assert torch.equal(oc, op)


def test_paged_entries_outside_the_pool(K):
    """A block-table entry outside the pool (-1, pool_pages): the encode writes nothing
    anywhere for those pages, and attention reads their records as zeros (the same output
    as a contiguous cache holding zero records there)."""
    wl = W.LLAMA_T32K
    alloc = [(64, 4, 64, 4)]
    B, g, cap, page, T = 1, 4, 1024, 128, 1000
    pps, pool_pages = cap // page, 10
    bk, bv = _bases(alloc, 31)
    table = H.block_table(7, B, pps, pool_pages)
    table[0, 2], table[0, 5] = -1, pool_pages
    bt = torch.from_numpy(table).cuda()
    lay_c = K.Layout(1, g, B, cap, alloc)
    lay_p = K.Layout(1, g, B, cap, alloc, page_tokens=page, pool_pages=pool_pages, block_table=bt)
    x = {t: W.tokens(wl, t, 0, 0, 0, T)[None, None] for t in "KV"}
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    ck_p = H.u32_dev(np.full(K.kv_cache_bytes(lay_p, 0) // 4, FILL, np.uint32))
    cv_p = H.u32_dev(np.full(K.kv_cache_bytes(lay_p, 1) // 4, FILL, np.uint32))
    K.kv_encode(lay_p, H.dev(x["K"]), H.dev(x["V"]), T, 0, pk, pv, ck_p, cv_p)
    gk_p = H.u32_host(ck_p)
    named = H.to_pool(np.zeros(K.kv_cache_bytes(lay_c, 0) // 4, np.uint32), [64], [4], B, cap, page, pool_pages,
                      table, fill=FILL)
    assert np.all(gk_p[named == FILL] == FILL)
    ck_c = H.u32_dev(H.from_pool(gk_p, [64], [4], B, cap, page, pool_pages, table))
    cv_c = H.u32_dev(H.from_pool(H.u32_host(cv_p), [64], [4], B, cap, page, pool_pages, table))
    q = H.dev(W.random_vectors(13, (B, g, 128)).astype(np.float16), torch.float16)
    ws = torch.zeros(K.kv_workspace_bytes(lay_c, T) // 4, dtype=torch.float32, device="cuda")
    out_c = torch.empty((B, g, 128), dtype=torch.float32, device="cuda")
    out_p = torch.empty_like(out_c)
    K.kv_attend_decode(lay_c, q, T, pk, pv, ck_c, cv_c, H.SCALE, out_c, ws)
    K.kv_attend_decode(lay_p, q, T, pk, pv, ck_p, cv_p, H.SCALE, out_p, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out_p).all()
    assert torch.equal(out_c, out_p)
