"""GPU parity of the attention-aware (NOVA-KV) key transform: keys encoded with
P_K = (M_q^(1/2) E)_r, the inverse folded into the query through
Q_K = (M_q^(-1/2) E)_r (kv_layout.query_basis_k), against the oracle's attention
over keys reconstructed as Q_K c^.  The records are the ordinary ones (the encode
basis is just another d x r matrix), so the encode parity tests cover them; here:
attention on oracle-built caches at several split sizes, the fused step against
append + attend, the 128K layer at full size (sampled units) and kv_decode of the
keys through Q_K."""
import numpy as np
import pytest

import harness as H
import workloads as W
from oracle import attention, codec

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


@pytest.fixture(scope="module")
def cal():
    return H.oracle_calibrate_nova(W.llama_t128k_nova(2.0))


def test_nova_attention_matches_oracle(K, cal):
    alloc, pk, qk, pv = cal
    wl = W.llama_t128k_nova(2.0)
    B, T, hkv, g = 2, 3000, wl.n_kv_heads, wl.group
    say(f"attention-aware keys: {alloc}")
    kv = {(t, b, h): W.tokens(wl, t, b, h, 0, T) for t in "KV" for b in range(B) for h in range(hkv)}
    ck_h, cv_h = H.oracle_cache(wl, alloc, pk, pv, B, T, T, kv=kv)
    q = W.random_vectors(61, (B, hkv * g, 128)).astype(np.float16)
    ref = attention.attend_cache(q.astype(np.float64), pk, pv, ck_h, cv_h, alloc, B, T, T, H.SCALE, query_bases=qk)
    lay = K.Layout(hkv, hkv * g, B, T, alloc, query_basis_k=True)
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    kb, vb = H.dev(H.key_pairs(pk, qk)), H.dev(codec.concat_bases(pv))
    for split in (0, 256):
        out = torch.full((B, hkv * g, 128), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(K.kv_workspace_bytes(lay, T, split) // 4, dtype=torch.float32, device="cuda")
        K.kv_attend_decode(lay, H.dev(q, torch.float16), T, kb, vb, ck, cv, H.SCALE, out, ws, split_tokens=split)
        torch.cuda.synchronize()
        err = H.rel_err_per_head(out.cpu().numpy(), ref)
        say(f"  split={split} max rel err {err:.3e}")
        assert err <= REL_TOL
    # the query basis matters: projecting with P_K instead gives another answer
    wrong = attention.attend_cache(q.astype(np.float64), pk, pv, ck_h, cv_h, alloc, B, T, T, H.SCALE)
    assert H.rel_err_per_head(wrong, ref) > 100 * REL_TOL


def test_nova_fused_step(K, cal):
    alloc, pk, qk, pv = cal
    wl = W.llama_t128k_nova(2.0)
    B, cap, T, hkv, g = 1, 2100, 2050, wl.n_kv_heads, wl.group
    kv = {(t, b, h): W.tokens(wl, t, b, h, 0, T) for t in "KV" for b in range(B) for h in range(hkv)}
    ck_h, cv_h = H.oracle_cache(wl, alloc, pk, pv, B, cap, T - 1, kv={k: x[: T - 1] for k, x in kv.items()})
    lay = K.Layout(hkv, hkv * g, B, cap, alloc, query_basis_k=True)
    kb, vb = H.dev(H.key_pairs(pk, qk)), H.dev(codec.concat_bases(pv))
    k1 = H.dev(np.stack([np.stack([kv["K", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), torch.float16)
    v1 = H.dev(np.stack([np.stack([kv["V", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), torch.float16)
    q = H.dev(W.random_vectors(67, (B, hkv * g, 128)).astype(np.float16), torch.float16)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    ck_f, cv_f = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_f = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    K.kv_append_attend_decode(lay, k1, v1, q, T, kb, vb, ck_f, cv_f, H.SCALE, out_f, ws)
    ck_s, cv_s = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_s = torch.empty_like(out_f)
    K.kv_append(lay, k1, v1, T - 1, kb, vb, ck_s, cv_s)
    K.kv_attend_decode(lay, q, T, kb, vb, ck_s, cv_s, H.SCALE, out_s, ws)
    torch.cuda.synchronize()
    assert torch.equal(ck_f, ck_s) and torch.equal(cv_f, cv_s)
    assert torch.equal(out_f, out_s)
    ok_h, ov_h = H.oracle_cache(wl, alloc, pk, pv, B, cap, T, kv=kv)
    gk, gv = H.u32_host(ck_f), H.u32_host(cv_f)
    rk, bits_k, rv, bits_v = zip(*alloc)
    for h in range(hkv):
        s0, s1, w = codec.record_slice(rk, bits_k, B, cap, h, 0, 0, T)
        H.compare_records(gk[s0:s1].reshape(T, w), ok_h[s0:s1].reshape(T, w), rk[h], bits_k[h], f"K h{h}",
                          kv["K", 0, h], pk[h])
        s0, s1, w = codec.record_slice(rv, bits_v, B, cap, h, 0, 0, T)
        H.compare_records(gv[s0:s1].reshape(T, w), ov_h[s0:s1].reshape(T, w), rv[h], bits_v[h], f"V h{h}",
                          kv["V", 0, h], pv[h])
    ref = attention.attend_cache(q.cpu().numpy().astype(np.float64), pk, pv, ok_h, ov_h, alloc, B, cap, T, H.SCALE,
                                 query_bases=qk)
    err = H.rel_err_per_head(out_f.cpu().numpy(), ref)
    say(f"  fused step max rel err {err:.3e}")
    assert err <= REL_TOL


def test_nova_full_size_128k_sampled_units(K, cal):
    alloc, pk, qk, pv = cal
    wl = W.llama_t128k_nova(2.0)
    T = wl.context + 1
    B, hkv, hq, g = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.group
    lay = K.Layout(hkv, hq, B, T, alloc, query_basis_k=True)
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    kb, vb = H.dev(H.key_pairs(pk, qk)), H.dev(codec.concat_bases(pv))
    for t0 in range(0, T, 1 << 15):
        n = min(1 << 15, T - t0)
        K.kv_encode(lay, H.dev(W.kv_array(wl, "K", t0, n)), H.dev(W.kv_array(wl, "V", t0, n)), n, t0, kb, vb, ck, cv)
    q = W.query_array(wl, 0)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q), T, kb, vb, ck, cv, H.SCALE, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bits_k, rv, bits_v = zip(*alloc)
    for b, h in [(0, 0), (B - 1, hkv - 1), (2, 3)]:
        xk = W.tokens(wl, "K", b, h, 0, T)
        xv = W.tokens(wl, "V", b, h, 0, T)
        rec_k = np.concatenate([codec.encode_tokens(xk[i:i + 16384], pk[h], bits_k[h]) for i in range(0, T, 16384)])
        rec_v = np.concatenate([codec.encode_tokens(xv[i:i + 16384], pv[h], bits_v[h]) for i in range(0, T, 16384)])
        s0, s1, w = codec.record_slice(rk, bits_k, B, T, h, b, 0, T)
        H.compare_records(gk[s0:s1].reshape(-1, w), rec_k, rk[h], bits_k[h], f"K b{b} h{h}", xk, pk[h])
        s0, s1, w = codec.record_slice(rv, bits_v, B, T, h, b, 0, T)
        H.compare_records(gv[s0:s1].reshape(-1, w), rec_v, rv[h], bits_v[h], f"V b{b} h{h}", xv, pv[h])
        ref = attention.attend_head_records(q[b, h * g:(h + 1) * g].astype(np.float64), pk[h], rec_k, rk[h],
                                            bits_k[h], pv[h], rec_v, rv[h], bits_v[h], H.SCALE, query_basis=qk[h])
        err = H.rel_err_per_head(got[b, h * g:(h + 1) * g], ref)
        say(f"  unit (b={b}, h={h}) {alloc[h]}: max rel err {err:.3e}")
        assert err <= REL_TOL


def test_nova_kv_decode_reconstructs_keys_through_the_query_basis(K, cal):
    alloc, pk, qk, pv = cal
    wl = W.llama_t128k_nova(2.0)
    B, T, hkv = 1, 300, wl.n_kv_heads
    ck_h, cv_h = H.oracle_cache(wl, alloc, pk, pv, B, T, T)
    lay = K.Layout(hkv, hkv, B, T, alloc, query_basis_k=True)
    out = torch.empty((B, hkv, T, 128), dtype=torch.float32, device="cuda")
    K.kv_decode(lay, 0, T, 0, H.dev(H.key_pairs(pk, qk)), H.u32_dev(ck_h), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rk, bits_k = [a[0] for a in alloc], [a[1] for a in alloc]
    for h in range(hkv):
        s0, s1, w = codec.record_slice(rk, bits_k, B, T, h, 0, 0, T)
        c = codec.decode_records(ck_h[s0:s1].reshape(T, w), rk[h], bits_k[h])
        Q = qk[h].astype(np.float64)
        bound = (rk[h] + 2) * 2.0 ** -24 * (np.abs(c) @ np.abs(Q).T) + 1e-30
        assert np.all(np.abs(got[0, h] - c @ Q.T) <= bound), f"head {h}"
