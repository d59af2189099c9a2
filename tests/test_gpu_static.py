"""GPU parity of header-free records (one fixed quantizer per head) and of the
record reconstruction kv_decode, against the CPU oracle.

* encode (prefill and append, fp16 and fp32 inputs): codes equal except at
  classified rounding ties, records outside the written range untouched, prefill
  records equal append records bit for bit (one-word records included);
* attention over oracle-built header-free caches: every format pair of the 64-
  and 128-bit budgets (their specialised kernels), odd widths and a layout with
  header-free keys beside headed values (the generic kernel): max relative error
  per (sequence, query head) <= 2e-3, for several split sizes;
* the fused append + attend step equals kv_append + kv_attend_decode bit for bit;
* the 128K LLaMA-shaped layer at 0.5 bits per dimension, header-free, at full
  size (sampled units);
* kv_decode of headed and header-free records against P (min + step * code).

The heads' fixed (min, step) come from the oracle (its static_scale of the
retained coordinates' common standard deviation).
"""
import numpy as np
import pytest

import harness as H
import workloads as W
from oracle import attention, codec, packing, transform

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


def _setup(alloc, seed, wl=W.LLAMA_T32K, keys=True, values=True):
    """Bases of random covariances, and fixed scales from the workload's own covariance."""
    bk, bv = [], []
    for h, (rk, _, rv, _) in enumerate(alloc):
        bk.append(transform.basis_for_head(W.random_covariance(seed + 10 + h, 128), rk,
                                           W.random_basis_signs(seed + h, rk)).astype(np.float32))
        bv.append(transform.basis_for_head(W.random_covariance(seed + 40 + h, 128), rv,
                                           W.random_basis_signs(seed + 50 + h, rv)).astype(np.float32))
    n = wl.n_kv_heads
    sk = H.oracle_static_scales([W.covariance(wl, "K", h % n) for h in range(len(alloc))], bk,
                                [a[1] for a in alloc]) if keys else None
    sv = H.oracle_static_scales([W.covariance(wl, "V", h % n) for h in range(len(alloc))], bv,
                                [a[3] for a in alloc]) if values else None
    return bk, bv, sk, sv


def _layout(K, alloc, g, B, cap, sk, sv):
    return K.Layout(len(alloc), len(alloc) * g, B, cap, alloc,
                    scale_k=None if sk is None else H.scale_words(sk),
                    scale_v=None if sv is None else H.scale_words(sv))


# ------------------------------------------------------------------ encode
def _check_records(got_all, x, alloc, bases, static, B, cap, pos0, n, tensor, sentinel=None):
    ranks = [a[0 if tensor == "K" else 2] for a in alloc]
    bits = [a[1 if tensor == "K" else 3] for a in alloc]
    flags = [static is not None] * len(alloc)
    for h in range(len(alloc)):
        for b in range(B):
            s0, s1, w = codec.record_slice(ranks, bits, B, cap, h, b, pos0, pos0 + n, flags)
            xh = x[b, h].astype(np.float64)
            got = got_all[s0:s1].reshape(n, w)
            what = f"{tensor} h{h} b{b}"
            if static is None:
                H.compare_records(got, codec.encode_tokens(xh, bases[h], bits[h]), ranks[h], bits[h], what, xh,
                                  bases[h])
            else:
                ref = codec.encode_tokens_static(xh, bases[h], bits[h], *static[h])
                H.compare_static_records(got, ref, ranks[h], bits[h], *static[h], what, xh, bases[h])
            if sentinel is not None:
                a0, _, _ = codec.record_slice(ranks, bits, B, cap, h, b, 0, 0, flags)
                a1, _, _ = codec.record_slice(ranks, bits, B, cap, h, b, cap, cap, flags)
                outside = np.concatenate([got_all[a0:s0], got_all[s1:a1]])
                assert np.all(outside == sentinel), f"{what}: write outside the range"


STATIC_ALLOC = [(16, 2, 128, 8), (32, 3, 64, 5), (64, 6, 32, 7), (128, 4, 16, 8), (16, 8, 16, 2)]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 17, 65, 1001])
def test_static_encode_matches_oracle(K, dtype, n):
    """Prefill (n > 1, matrix-core projection) and append (n = 1) of header-free records,
    one-word records (16, 2) included; nothing outside positions pos0 .. pos0+n-1 written."""
    say(f"header-free encode {dtype} n={n}")
    alloc = STATIC_ALLOC
    wl = W.LLAMA_T32K
    bk, bv, sk, sv = _setup(alloc, 3)
    B, pos0 = 2, 37
    cap = pos0 + n + 5
    lay = _layout(K, alloc, 1, B, cap, sk, sv)
    sentinel = np.uint32(0xA5A5A5A5)
    ck = H.u32_dev(np.full(K.kv_cache_bytes(lay, 0) // 4, sentinel, np.uint32))
    cv = H.u32_dev(np.full(K.kv_cache_bytes(lay, 1) // 4, sentinel, np.uint32))
    x = {t: np.stack([np.stack([W.tokens(wl, t, b, h % wl.n_kv_heads, 11, n, dtype) for h in range(len(alloc))])
                      for b in range(B)]) for t in "KV"}
    tdt = torch.float32 if dtype == "f32" else torch.float16
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    if n == 1:
        K.kv_append(lay, H.dev(x["K"][:, :, 0], tdt), H.dev(x["V"][:, :, 0], tdt), pos0, pk, pv, ck, cv)
    else:
        K.kv_encode(lay, H.dev(x["K"], tdt), H.dev(x["V"], tdt), n, pos0, pk, pv, ck, cv)
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    _check_records(gk, x["K"], alloc, bk, sk, B, cap, pos0, n, "K", sentinel)
    _check_records(gv, x["V"], alloc, bv, sv, B, cap, pos0, n, "V", sentinel)


def test_static_prefill_records_equal_append_records(K):
    say("header-free prefill records == append records")
    alloc = STATIC_ALLOC
    wl = W.LLAMA_T32K
    bk, bv, sk, sv = _setup(alloc, 7)
    B, n = 2, 200
    lay = _layout(K, alloc, 1, B, n, sk, sv)
    x = {t: np.stack([np.stack([W.tokens(wl, t, b, h % wl.n_kv_heads, 0, n) for h in range(len(alloc))])
                      for b in range(B)]) for t in "KV"}
    kd, vd = H.dev(x["K"], torch.float16), H.dev(x["V"], torch.float16)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    ck_e = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv_e = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    ck_a, cv_a = torch.zeros_like(ck_e), torch.zeros_like(cv_e)
    K.kv_encode(lay, kd, vd, n, 0, pk, pv, ck_e, cv_e)
    for t in range(n):
        K.kv_append(lay, kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), t, pk, pv, ck_a, cv_a)
    torch.cuda.synchronize()
    assert torch.equal(ck_e, ck_a) and torch.equal(cv_e, cv_a)


# ------------------------------------------------------------------ attention
def _attention_case(K, alloc, bk, bv, sk, sv, B, g, cap, T, splits, seed=0, wl=W.LLAMA_T32K):
    hkv = len(alloc)
    kv = {(t, b, h): W.tokens(wl, t, b, h % wl.n_kv_heads, 0, T) for t in "KV" for b in range(B) for h in range(hkv)}
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T, kv=kv, static_k=sk, static_v=sv)
    q = W.random_vectors(seed, (B, hkv * g, 128)).astype(np.float16)
    ref = attention.attend_cache(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, B, cap, T, H.SCALE, sk, sv)
    lay = _layout(K, alloc, g, B, cap, sk, sv)
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    qd = H.dev(q, torch.float16)
    outs = {}
    for split in splits:
        out = torch.full((B, hkv * g, 128), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(K.kv_workspace_bytes(lay, T, split) // 4, dtype=torch.float32, device="cuda")
        K.kv_attend_decode(lay, qd, T, pk, pv, ck, cv, H.SCALE, out, ws, split_tokens=split)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        err = H.rel_err_per_head(got, ref)
        say(f"  split={split} max rel err {err:.3e}")
        assert err <= REL_TOL
        outs[split] = got
    return outs


def _budget_formats(budget_bits):
    return [(r, min(8, budget_bits // r)) for r in (16, 32, 64, 128) if min(8, budget_bits // r) >= 2]


@pytest.mark.parametrize("budget", [64, 128])
@pytest.mark.parametrize("g", [4, 7])
def test_static_attention_every_format_pair_of_a_budget(K, budget, g):
    fm = _budget_formats(budget)
    alloc = [(rk, bk_, rv, bv_) for (rk, bk_) in fm for (rv, bv_) in fm]
    say(f"header-free attention, budget {budget} bits, g={g}, {len(alloc)} heads")
    bk, bv, sk, sv = _setup(alloc, 31 + budget + g)
    _attention_case(K, alloc, bk, bv, sk, sv, 1, g, 800, 777, [0, 256])


@pytest.mark.parametrize("which", ["both", "keys", "values"])
def test_static_attention_generic_kernel(K, which):
    """Odd widths (the generic kernel), with header-free keys and values, keys only, or
    values only (headed records of the other tensor)."""
    say(f"header-free attention, generic kernel, {which}")
    alloc = STATIC_ALLOC
    bk, bv, sk, sv = _setup(alloc, 19, keys=which != "values", values=which != "keys")
    _attention_case(K, alloc, bk, bv, sk, sv, 2, 4, 2100, 2000, [0, 256], seed=5)


@pytest.mark.parametrize("T", [1, 255, 257])
def test_static_attention_short_contexts(K, T):
    say(f"header-free attention T={T}")
    alloc = [(16, 4, 32, 2), (32, 2, 16, 4)]
    bk, bv, sk, sv = _setup(alloc, 23)
    _attention_case(K, alloc, bk, bv, sk, sv, 2, 4, T, T, [0])


def test_static_fused_append_attend(K):
    say("header-free fused append + attend")
    alloc = [(16, 4, 32, 2), (32, 2, 16, 4), (16, 8, 64, 2)]
    wl = W.LLAMA_T32K
    bk, bv, sk, sv = _setup(alloc, 29)
    B, g, cap, T = 2, 4, 1300, 1234
    hkv = len(alloc)
    kv = {(t, b, h): W.tokens(wl, t, b, h, 0, T) for t in "KV" for b in range(B) for h in range(hkv)}
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T - 1, kv={k: x[: T - 1] for k, x in kv.items()},
                                static_k=sk, static_v=sv)
    lay = _layout(K, alloc, g, B, cap, sk, sv)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    k1 = H.dev(np.stack([np.stack([kv["K", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), torch.float16)
    v1 = H.dev(np.stack([np.stack([kv["V", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), torch.float16)
    q = H.dev(W.random_vectors(47, (B, hkv * g, 128)).astype(np.float16), torch.float16)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    ck_f, cv_f = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_f = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    K.kv_append_attend_decode(lay, k1, v1, q, T, pk, pv, ck_f, cv_f, H.SCALE, out_f, ws)
    ck_s, cv_s = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_s = torch.empty_like(out_f)
    K.kv_append(lay, k1, v1, T - 1, pk, pv, ck_s, cv_s)
    K.kv_attend_decode(lay, q, T, pk, pv, ck_s, cv_s, H.SCALE, out_s, ws)
    torch.cuda.synchronize()
    assert torch.equal(ck_f, ck_s) and torch.equal(cv_f, cv_s)
    assert torch.equal(out_f, out_s)
    ok_h, ov_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T, kv=kv, static_k=sk, static_v=sv)
    gk, gv = H.u32_host(ck_f), H.u32_host(cv_f)
    x = {t: np.stack([np.stack([kv[t, b, h] for h in range(hkv)]) for b in range(B)]) for t in "KV"}
    _check_records(gk, x["K"], alloc, bk, sk, B, cap, 0, T, "K")
    _check_records(gv, x["V"], alloc, bv, sv, B, cap, 0, T, "V")
    ref = attention.attend_cache(q.cpu().numpy().astype(np.float64), bk, bv, ok_h, ov_h, alloc, B, cap, T, H.SCALE,
                                 sk, sv)
    err = H.rel_err_per_head(out_f.cpu().numpy(), ref)
    say(f"  max rel err {err:.3e}")
    assert err <= REL_TOL


def test_static_full_size_128k_half_bit(K):
    """The 128K LLaMA-shaped layer at 0.5 bits per dimension with header-free records
    (8 bytes per record instead of 12), encoded on the GPU at full size and attended in
    the benchmark's launch configuration; sampled units re-encoded and attended by the
    oracle."""
    wl = W.llama_t128k(0.5)
    T = wl.context + 1
    B, hkv, hq, g = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.group
    alloc, bk, bv = H.oracle_calibrate(wl)
    sk = H.oracle_static_scales([W.covariance(wl, "K", h) for h in range(hkv)], bk, [a[1] for a in alloc])
    sv = H.oracle_static_scales([W.covariance(wl, "V", h) for h in range(hkv)], bv, [a[3] for a in alloc])
    say(f"header-free full size {wl.name}: {alloc}")
    lay = _layout(K, alloc, g, B, T, sk, sv)
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    for t0 in range(0, T, 1 << 15):
        n = min(1 << 15, T - t0)
        K.kv_encode(lay, H.dev(W.kv_array(wl, "K", t0, n)), H.dev(W.kv_array(wl, "V", t0, n)), n, t0, pk, pv, ck, cv)
    q = W.query_array(wl, 0)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q), T, pk, pv, ck, cv, H.SCALE, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bits_k, rv, bits_v = zip(*alloc)
    fl = [True] * hkv
    for b, h in [(0, 0), (B - 1, hkv - 1), (1, hkv // 2)]:
        xk = W.tokens(wl, "K", b, h, 0, T)
        xv = W.tokens(wl, "V", b, h, 0, T)
        rec_k = np.concatenate([codec.encode_tokens_static(xk[i:i + 16384], bk[h], bits_k[h], *sk[h])
                                for i in range(0, T, 16384)])
        rec_v = np.concatenate([codec.encode_tokens_static(xv[i:i + 16384], bv[h], bits_v[h], *sv[h])
                                for i in range(0, T, 16384)])
        s0, s1, w = codec.record_slice(rk, bits_k, B, T, h, b, 0, T, fl)
        fk = H.compare_static_records(gk[s0:s1].reshape(-1, w), rec_k, rk[h], bits_k[h], *sk[h], f"K b{b} h{h}",
                                      xk, bk[h])
        s0, s1, w = codec.record_slice(rv, bits_v, B, T, h, b, 0, T, fl)
        fv = H.compare_static_records(gv[s0:s1].reshape(-1, w), rec_v, rv[h], bits_v[h], *sv[h], f"V b{b} h{h}",
                                      xv, bv[h])
        ref = attention.attend_head_records(q[b, h * g:(h + 1) * g].astype(np.float64), bk[h], rec_k, rk[h],
                                            bits_k[h], bv[h], rec_v, rv[h], bits_v[h], H.SCALE, sk[h], sv[h])
        err = H.rel_err_per_head(got[b, h * g:(h + 1) * g], ref)
        say(f"  unit (b={b}, h={h}) {alloc[h]}: code mismatch K {fk:.1e} V {fv:.1e}, max rel err {err:.3e}")
        assert err <= REL_TOL


# ------------------------------------------------------------------ reconstruction
@pytest.mark.parametrize("static", [False, True])
def test_kv_decode_matches_oracle(K, static):
    """x^ = P (min + step * code) of every stored token, against the oracle's float64
    reconstruction within the float32 bound: r fused multiply-adds in order, each
    rounded once (gamma_r <= (r + 1) 2^-24 of sum_j |P_ij c^_j|), after one rounding of
    each dequantized coordinate (2^-24 more)."""
    say(f"kv_decode, header-free {static}")
    alloc = STATIC_ALLOC
    bk, bv, sk, sv = _setup(alloc, 37)
    if not static:
        sk = sv = None
    B, cap, T, pos0, n = 2, 600, 600, 13, 555
    wl = W.LLAMA_T32K
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T, static_k=sk, static_v=sv,
                                kv={(t, b, h): W.tokens(wl, t, b, h % 8, 0, T) for t in "KV" for b in range(B)
                                    for h in range(len(alloc))})
    lay = _layout(K, alloc, 1, B, cap, sk, sv)
    for which, cache, bases, st in ((0, ck_h, bk, sk), (1, cv_h, bv, sv)):
        out = torch.full((B, len(alloc), n, 128), float("nan"), dtype=torch.float32, device="cuda")
        K.kv_decode(lay, which, n, pos0, H.dev(codec.concat_bases(bases)), H.u32_dev(cache), out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ranks = [a[2 * which] for a in alloc]
        bits = [a[2 * which + 1] for a in alloc]
        flags = [st is not None] * len(alloc)
        for h in range(len(alloc)):
            for b in range(B):
                s0, s1, w = codec.record_slice(ranks, bits, B, cap, h, b, pos0, pos0 + n, flags)
                rec = cache[s0:s1].reshape(n, w)
                c = (codec.decode_records(rec, ranks[h], bits[h]) if st is None
                     else codec.decode_records_static(rec, ranks[h], bits[h], *st[h]))
                P = np.asarray(bases[h], np.float64)
                ref = c @ P.T
                bound = (ranks[h] + 2) * 2.0 ** -24 * (np.abs(c) @ np.abs(P).T) + 1e-30
                assert np.all(np.abs(got[b, h] - ref) <= bound), f"tensor {which} h{h} b{b}"
