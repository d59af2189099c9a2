"""GPU parity of decode attention over keys compressed before RoPE
(kv_attend_decode_rope, kv_append_attend_decode_rope) against the oracle.

The caches hold the oracle's records of unrotated keys; the oracle reconstructs
each key, turns it by its position and runs textbook softmax attention.  The bar
is the attention bar: max over (sequence, query head) of
||o_gpu - o_ref||_inf / ||o_ref||_inf <= 2e-3, at several split sizes, ranks,
widths, group sizes, header-free keys, short and ragged contexts, and sampled
units of the 128K LLaMA-shaped layer.  The fused step equals append + attend bit
for bit.
"""
import numpy as np
import pytest

import harness as H
import workloads as W
from oracle import codec, rope, transform

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

REL_TOL = 2e-3


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_04_amd as K
    K.kv_record_words(16, 2)  # loads the library (fails loudly if it is missing)
    return K


def say(*a):
    print(*a, flush=True)


def _bases(alloc, seed):
    bk, bv = [], []
    for h, (rk, _, rv, _) in enumerate(alloc):
        bk.append(transform.basis_for_head(W.random_covariance(seed + 10 + h, 128), rk,
                                           W.random_basis_signs(seed + h, rk)).astype(np.float32))
        bv.append(transform.basis_for_head(W.random_covariance(seed + 40 + h, 128), rv,
                                           W.random_basis_signs(seed + 50 + h, rv)).astype(np.float32))
    return bk, bv


def _rope_attend(K, lay, q, T, bk, bv, ck, cv, inv_freq, split=0):
    B, hq = lay.batch, lay.n_q_heads
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(K.kv_workspace_bytes_rope(lay, T, split) // 4, dtype=torch.float32, device="cuda")
    K.kv_attend_decode_rope(lay, q, T, H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv)), ck, cv,
                            H.SCALE, torch.from_numpy(np.asarray(inv_freq, np.float64)).cuda(), out, ws,
                            split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _case(K, alloc, g, batch, cap, T, splits, inv_freq, seed=0, static=False, qdtype=np.float16,
          wl=W.LLAMA_T32K):
    hkv = len(alloc)
    bk, bv = _bases(alloc, seed)
    kv = {(t, b, h): W.tokens(wl, t, b, h % wl.n_kv_heads, 0, T) for t in "KV" for b in range(batch)
          for h in range(hkv)}
    st_k = None
    if static:
        covs = [np.cov(np.concatenate([kv[("K", b, h)] for b in range(batch)]).T) for h in range(hkv)]
        st_k = H.oracle_static_scales(covs, bk, [a[1] for a in alloc])
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, batch, cap, T, kv=kv, static_k=st_k)
    q = W.random_vectors(seed + 3, (batch, hkv * g, 128)).astype(qdtype)
    ref = rope.attend_cache_rope(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, batch, cap, T, H.SCALE,
                                 inv_freq, static_k=st_k)
    lay = K.Layout(hkv, hkv * g, batch, cap, alloc, scale_k=None if st_k is None else H.scale_words(st_k))
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    qd = torch.from_numpy(q).cuda()
    errs = []
    for split in splits:
        got = _rope_attend(K, lay, qd, T, bk, bv, ck, cv, inv_freq, split)
        assert np.isfinite(got).all()
        err = H.rel_err_per_head(got, ref)
        say(f"  split={split} max rel err {err:.3e}")
        assert err <= REL_TOL
        errs.append(err)
    return errs


ROFORMER = rope.default_inv_freq(128, 10000.0)
LLAMA3 = rope.default_inv_freq(128, 500000.0)


@pytest.mark.parametrize("alloc,g", [
    ([(128, 2, 128, 2), (64, 4, 64, 4)], 4),
    ([(32, 8, 64, 4), (16, 4, 128, 2)], 4),
    ([(64, 3, 32, 5), (32, 6, 16, 7)], 2),
    ([(128, 2, 16, 6)], 7),
    ([(64, 4, 128, 4), (128, 8, 32, 8)], 8),
    ([(16, 8, 64, 4)], 1),
], ids=["r128b2-r64b4-g4", "r32b8-r16b4-g4", "odd-widths-g2", "qwen-mixed-g7", "r128b8-g8", "r16-g1"])
def test_rope_attention_matches_oracle(K, alloc, g):
    say(f"rope attention {alloc} g={g}")
    _case(K, alloc, g, 2, 3100, 3000, [0, 256, 768], ROFORMER, seed=len(alloc) * 7 + g)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 257, 1000])
def test_rope_short_and_ragged_contexts(K, T):
    say(f"rope attention T={T}")
    _case(K, [(64, 4, 32, 8), (128, 2, 64, 4)], 4, 2, T, T, [0, 256], LLAMA3, seed=T)


def test_rope_header_free_keys(K):
    say("rope attention, header-free keys")
    _case(K, [(128, 2, 128, 2), (64, 4, 64, 4)], 4, 2, 2100, 2000, [0, 512], ROFORMER, seed=5, static=True)


def test_rope_float32_query_and_large_positions(K):
    """fp32 queries and positions up to 40000 (angles far beyond 2 pi for the fast pairs)."""
    say("rope attention, fp32 query, 40000 tokens")
    _case(K, [(64, 4, 64, 4)], 4, 1, 40000, 40000, [0], LLAMA3, seed=9, qdtype=np.float32)


def test_rope_zero_frequencies_match_plain_attention(K):
    """With every inverse frequency zero no key turns: the result is plain attention
    over the same records (both paths against the same oracle value)."""
    say("rope attention, zero frequencies")
    _case(K, [(128, 2, 128, 2), (32, 8, 64, 4)], 4, 2, 1500, 1500, [0], np.zeros(64), seed=11)


def test_rope_fused_step_equals_append_then_attend(K):
    """kv_append_attend_decode_rope writes kv_append's records and returns
    kv_attend_decode_rope's output over them, bit for bit."""
    say("rope fused append + attend")
    alloc = [(128, 2, 128, 2), (64, 4, 32, 8)]
    B, g, cap, T = 2, 4, 2100, 2049
    wl = W.LLAMA_T32K
    bk, bv = _bases(alloc, 21)
    lay = K.Layout(2, 2 * g, B, cap, alloc)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    kx = np.stack([np.stack([W.tokens(wl, "K", b, h, 0, T) for h in range(2)]) for b in range(B)])
    vx = np.stack([np.stack([W.tokens(wl, "V", b, h, 0, T) for h in range(2)]) for b in range(B)])
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    K.kv_encode(lay, H.dev(kx[:, :, :T - 1], torch.float16), H.dev(vx[:, :, :T - 1], torch.float16), T - 1, 0, pk,
                pv, ck, cv)
    k1, v1 = H.dev(kx[:, :, T - 1], torch.float16), H.dev(vx[:, :, T - 1], torch.float16)
    q = torch.from_numpy(W.random_vectors(23, (B, 2 * g, 128)).astype(np.float16)).cuda()
    th = torch.from_numpy(LLAMA3).cuda()
    ws = torch.zeros(K.kv_workspace_bytes_rope(lay, T) // 4, dtype=torch.float32, device="cuda")
    ck2, cv2 = ck.clone(), cv.clone()
    out = torch.empty((B, 2 * g, 128), dtype=torch.float32, device="cuda")
    K.kv_append_attend_decode_rope(lay, k1, v1, q, T, pk, pv, ck, cv, H.SCALE, th, out, ws)
    out2 = torch.empty_like(out)
    K.kv_append(lay, k1, v1, T - 1, pk, pv, ck2, cv2)
    K.kv_attend_decode_rope(lay, q, T, pk, pv, ck2, cv2, H.SCALE, th, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(ck, ck2) and torch.equal(cv, cv2)
    assert torch.equal(out, out2)
    ref = rope.attend_cache_rope(q.cpu().numpy().astype(np.float64), bk, bv, H.u32_host(ck), H.u32_host(cv), alloc,
                                 B, cap, T, H.SCALE, LLAMA3)
    err = H.rel_err_per_head(out.cpu().numpy(), ref)
    say(f"  max rel err {err:.3e}")
    assert err <= REL_TOL


def test_rope_full_size_llama_t128k_sampled_units(K):
    """The LLaMA-shaped 128K layer at 2 bits per dimension (batch 4, 32 query heads
    over 8 KV heads, 131073 tokens, the default split plan): GPU prefill encode, then
    attention over pre-RoPE keys; three (sequence, KV head) units checked against the
    oracle over all their tokens."""
    wl = W.llama_t128k(2.0)
    T = wl.context + 1
    B, hkv, g = wl.batch, wl.n_kv_heads, wl.group
    alloc, bk, bv = H.oracle_calibrate(wl)
    lay = K.Layout(hkv, wl.n_q_heads, B, T, alloc)
    ns = K.kv_workspace_bytes_rope(lay, T)
    say(f"rope full size {wl.name}: {alloc}")
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    kx = W.kv_array(wl, "K", 0, T)
    vx = W.kv_array(wl, "V", 0, T)
    K.kv_encode(lay, H.dev(kx), H.dev(vx), T, 0, pk, pv, ck, cv)
    q = W.query_array(wl, 0)
    th = rope.default_inv_freq(128, 500000.0)
    out = torch.empty((B, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(ns // 4, dtype=torch.float32, device="cuda")
    K.kv_attend_decode_rope(lay, H.dev(q), T, pk, pv, ck, cv, H.SCALE, torch.from_numpy(th).cuda(), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bits_k, rv, bits_v = zip(*alloc)
    worst = 0.0
    for b, h in [(0, 0), (1, 5), (3, 7)]:
        s0, s1, w = codec.record_slice(rk, bits_k, B, T, h, b, 0, T)
        ckh = codec.decode_records(gk[s0:s1].reshape(T, w), rk[h], bits_k[h])
        s0, s1, w = codec.record_slice(rv, bits_v, B, T, h, b, 0, T)
        cvh = codec.decode_records(gv[s0:s1].reshape(T, w), rv[h], bits_v[h])
        for i in range(g):
            ref = rope.attend_coords_rope(q[b, h * g + i].astype(np.float64), bk[h], ckh, bv[h], cvh, H.SCALE,
                                          np.arange(T), th)
            err = float(np.abs(got[b, h * g + i] - ref).max() / np.abs(ref).max())
            worst = max(worst, err)
            assert err <= REL_TOL, (b, h, i, err)
    say(f"  sampled units: max rel err {worst:.3e}")
