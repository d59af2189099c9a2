"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

* quantize/pack and unpack: bit-exact for every (rank, bits) and the edge cases;
* encode / append: headers exact, codes equal except at rounding ties (<= 1e-5
  of codes, each off by one), records outside the written range untouched;
* attention over an identical (oracle-built) cache: max over (sequence, query
  head) of ||o_gpu - o_ref||_inf / ||o_ref||_inf <= 2e-3, for several split sizes;
* end-to-end (GPU encode -> GPU attend vs oracle encode -> oracle attend).
"""
import numpy as np
import pytest

import harness as H
import workloads as W
from oracle import attention, codec, packing, quantizer, transform

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

REL_TOL = 2e-3        # attention output, max relative error per (sequence, query head)


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_04_amd as K
    K.kv_record_words(16, 2)  # loads the library (fails loudly if it is missing)
    return K


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ quantize / pack / unpack
def _edge_rows(r, b):
    L = 2 ** b - 1
    rows = []
    rows.append(np.full(r, 0.3))                                   # all equal: step 0
    tie = np.zeros(r)
    tie[1] = L
    tie[2:] = (np.arange(r - 2) % L) + 0.5                          # exact half-way values
    rows.append(tie)
    rows.append(-np.abs(np.linspace(0.0, 5.0, r)))                 # negative values
    mid = 1.0 + 2.0 ** -11                                         # min exactly between two fp16 values
    rows.append(np.linspace(mid, mid + 3.0, r))
    rows.append(np.linspace(1e-6, 3e-6, r))                        # subnormal fp16 step
    rows.append(np.linspace(-3e4, 3e4, r))                         # large range
    big = np.zeros(r)
    big[0] = 1.0
    rows.append(big)                                               # one non-zero coordinate
    return np.array(rows, np.float32)


@pytest.mark.parametrize("r", [16, 32, 64, 128])
@pytest.mark.parametrize("b", list(range(2, 9)))
def test_quantize_pack_bit_exact(K, r, b):
    say(f"quantize_pack r={r} b={b}")
    x = np.concatenate([W.random_coords(r * 16 + b, 1037, r), _edge_rows(r, b)])
    n, w = len(x), packing.record_words(r, b)
    rec = torch.empty((n, w), dtype=torch.int32, device="cuda")
    K.kv_quantize_pack(H.dev(x), r, b, rec)
    got = H.u32_host(rec)
    mu, sg, codes = quantizer.quantize(x.astype(np.float64), b)
    ref = packing.pack(mu, sg, codes, b)
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} records differ, first token {bad[:5]}"


@pytest.mark.parametrize("r,b", [(16, 2), (16, 3), (32, 5), (64, 6), (128, 7), (128, 8), (64, 4)])
def test_unpack_bit_exact(K, r, b):
    say(f"unpack r={r} b={b}")
    n = 777
    codes = W.random_codes(5 + r + b, n, r, b)
    x = W.random_coords(77, n, r).astype(np.float64)
    mu, sg, _ = quantizer.quantize(x, b)
    rec = packing.pack(mu, sg, codes, b)
    ms = torch.empty((n, 2), dtype=torch.int16, device="cuda")
    cg = torch.empty((n, r), dtype=torch.uint8, device="cuda")
    K.kv_unpack(H.u32_dev(rec), n, r, b, ms, cg)
    torch.cuda.synchronize()
    ms_h = ms.cpu().numpy().view(np.uint16)
    assert np.array_equal(ms_h[:, 0], quantizer.fp16_bits(mu).astype(np.uint16))
    assert np.array_equal(ms_h[:, 1], quantizer.fp16_bits(sg).astype(np.uint16))
    assert np.array_equal(cg.cpu().numpy().astype(np.int64), codes)


# ------------------------------------------------------------------ layouts used below
MIXED_ALLOC = [(16, 2, 128, 8), (32, 3, 64, 5), (64, 6, 32, 7), (128, 4, 16, 8)]


def _mixed_bases(alloc, seed=0):
    bk, bv = [], []
    for h, (rk, _, rv, _) in enumerate(alloc):
        ck = W.random_covariance(seed + 10 + h, 128)
        cv = W.random_covariance(seed + 40 + h, 128)
        bk.append(transform.basis_for_head(ck, rk, W.random_basis_signs(seed + h, rk)).astype(np.float32))
        bv.append(transform.basis_for_head(cv, rv, W.random_basis_signs(seed + 50 + h, rv)).astype(np.float32))
    return bk, bv


def _encode_case(K, wl_tokens, alloc, bases_k, bases_v, batch, cap, pos0, n, dtype):
    hkv = len(alloc)
    lay = K.Layout(hkv, hkv, batch, cap, alloc)
    sentinel = np.uint32(0xA5A5A5A5)
    nk = K.kv_cache_bytes(lay, 0) // 4
    nv = K.kv_cache_bytes(lay, 1) // 4
    ck = H.u32_dev(np.full(nk, sentinel, np.uint32))
    cv = H.u32_dev(np.full(nv, sentinel, np.uint32))
    kx = np.stack([np.stack([wl_tokens("K", b, h, n) for h in range(hkv)]) for b in range(batch)])
    vx = np.stack([np.stack([wl_tokens("V", b, h, n) for h in range(hkv)]) for b in range(batch)])
    tdt = torch.float32 if dtype == "f32" else torch.float16
    K.kv_encode(lay, H.dev(kx, tdt), H.dev(vx, tdt), n, pos0, H.dev(codec.concat_bases(bases_k)),
                H.dev(codec.concat_bases(bases_v)), ck, cv)
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bk, rv, bv = zip(*alloc)
    for tensor, got_all, ranks, bits, bases, x in (("K", gk, rk, bk, bases_k, kx), ("V", gv, rv, bv, bases_v, vx)):
        for h in range(hkv):
            for b in range(batch):
                s0, s1, w = codec.record_slice(ranks, bits, batch, cap, h, b, pos0, pos0 + n)
                ref = codec.encode_tokens(x[b, h].astype(np.float64), bases[h], bits[h])
                H.compare_records(got_all[s0:s1].reshape(n, w), ref, ranks[h], bits[h], f"{tensor} h{h} b{b}",
                                 x[b, h], bases[h])
                a0, _, _ = codec.record_slice(ranks, bits, batch, cap, h, b, 0, 0)
                a1, _, _ = codec.record_slice(ranks, bits, batch, cap, h, b, cap, cap)
                outside = np.concatenate([got_all[a0:s0], got_all[s1:a1]])
                assert np.all(outside == sentinel), f"{tensor} h{h} b{b}: write outside the range"
    return lay


def test_encode_tiny_fp32_matches_oracle(K):
    say("encode tiny-1head-T4096 fp32")
    wl = W.TINY
    alloc, bk, bv = H.oracle_calibrate(wl)
    _encode_case(K, lambda t, b, h, n: W.tokens(wl, t, b, h, 0, n), alloc, bk, bv, 1, 4096, 0, 4096, "f32")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_encode_mixed_allocation_matches_oracle(K, dtype):
    say(f"encode mixed allocation {dtype}")
    wl = W.LLAMA_T32K
    bk, bv = _mixed_bases(MIXED_ALLOC)
    _encode_case(K, lambda t, b, h, n: W.tokens(wl, t, b, h, 0, n, dtype), MIXED_ALLOC, bk, bv,
                 2, 1100, 37, 1001, dtype)


def test_encode_mixed_ranks_stream_ordered(K):
    """A layout with four ranks encodes them in four launches on the caller's stream.
    What that stream runs next must see every record: a clone enqueued right behind
    each encode on a non-default stream (no device-wide synchronisation in between)
    equals the records encoded on the default stream, and so does a captured graph of
    the encode, replayed three times with eager work between the replays."""
    say("encode mixed ranks: stream order, graph replays")
    wl = W.LLAMA_T32K
    bk, bv = _mixed_bases(MIXED_ALLOC)
    hkv, batch, cap, n = len(MIXED_ALLOC), 2, 1100, 1001
    lay = K.Layout(hkv, hkv, batch, cap, MIXED_ALLOC)
    kx = np.stack([np.stack([W.tokens(wl, "K", b, h, 0, n, "f16") for h in range(hkv)]) for b in range(batch)])
    vx = np.stack([np.stack([W.tokens(wl, "V", b, h, 0, n, "f16") for h in range(hkv)]) for b in range(batch)])
    kd, vd = H.dev(kx, torch.float16), H.dev(vx, torch.float16)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    nk, nv = K.kv_cache_bytes(lay, 0) // 4, K.kv_cache_bytes(lay, 1) // 4
    dev = torch.device("cuda")
    ref_k = torch.zeros(nk, dtype=torch.int32, device=dev)
    ref_v = torch.zeros(nv, dtype=torch.int32, device=dev)
    K.kv_encode(lay, kd, vd, n, 0, pk, pv, ref_k, ref_v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    copies = []
    with torch.cuda.stream(side):
        for _ in range(3):
            ck = torch.zeros(nk, dtype=torch.int32, device=dev)
            cv = torch.zeros(nv, dtype=torch.int32, device=dev)
            K.kv_encode(lay, kd, vd, n, 0, pk, pv, ck, cv)
            copies.append((ck.clone(), cv.clone()))
    side.synchronize()
    for i, (ck, cv) in enumerate(copies):
        assert torch.equal(ck, ref_k) and torch.equal(cv, ref_v), f"stream-ordered copy {i} differs"
    gk = torch.zeros(nk, dtype=torch.int32, device=dev)
    gv = torch.zeros(nv, dtype=torch.int32, device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        K.kv_encode(lay, kd, vd, n, 0, pk, pv, gk, gv)
    for rep in range(3):
        gk.zero_()
        gv.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gk, ref_k) and torch.equal(gv, ref_v), f"graph replay {rep} differs"


@pytest.mark.parametrize("n", [2, 15, 16, 17, 63, 65, 129, 257, 513])
def test_encode_ragged_token_counts(K, n):
    """Token counts around the encoder's 16-token blocks and 64/128-token tiles; nothing
    outside positions pos0 .. pos0+n-1 is written."""
    say(f"encode n={n}")
    wl = W.LLAMA_T32K
    alloc = [(128, 2, 16, 8), (64, 5, 32, 3)]
    bk, bv = _mixed_bases(alloc, seed=7)
    _encode_case(K, lambda t, b, h, n_: W.tokens(wl, t, b, h, 11, n_), alloc, bk, bv, 2, n + 9, 9, n, "f16")


def _degenerate_tokens(n, seed, dtype):
    """Tokens at the edges of the encoder's input domain, in a repeating pattern: zero
    vectors (all coordinates 0: step 0, every code 0), constant vectors, one non-zero
    dimension, repeated identical tokens, and tokens of norm 60000 (the documented
    limit is ||x||_2 max_j ||P_j||_2 <= 65504; here the bases are orthonormal)."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(n):
        kind = i % 6
        if kind == 0:
            x = np.zeros(128)
        elif kind == 1:
            x = np.full(128, 0.75 * (1 + i % 5))
        elif kind == 2:
            x = np.zeros(128)
            x[(7 * i) % 128] = 1000.0 * (-1) ** i
        elif kind == 3:
            x = np.linspace(-1.0, 1.0, 128) * 3.0  # the same token each time
        else:
            z = rng.standard_normal(128)
            x = z * (60000.0 / np.linalg.norm(z)) if kind == 4 else z * 1e-3
        rows.append(x)
    return np.array(rows).astype(np.float32 if dtype == "f32" else np.float16)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_encode_degenerate_tokens(K, dtype):
    """Zero, constant, one-hot, repeated, tiny and near-limit tokens: prefill records
    against the oracle (headers exact, codes up to classified ties)."""
    say(f"encode degenerate tokens {dtype}")
    alloc = [(16, 2, 128, 8), (64, 4, 32, 5), (128, 3, 64, 7)]
    bk, bv = _mixed_bases(alloc, seed=83)
    _encode_case(K, lambda t, b, h, n: _degenerate_tokens(n, 1000 * b + 10 * h + (t == "V"), dtype), alloc, bk, bv,
                 2, 140, 6, 130, dtype)


def test_attention_identical_keys_is_the_value_mean(K):
    """Every key zero: all scores equal, so each query head's output is the plain mean
    of its KV head's reconstructed values (a closed form), for GPU and oracle alike."""
    say("attention over identical keys")
    alloc = [(64, 4, 128, 2), (32, 8, 64, 4)]
    bk, bv = _mixed_bases(alloc, seed=89)
    wl, B, g, T = W.LLAMA_T32K, 2, 4, 700
    kv = {}
    for b in range(B):
        for h in range(len(alloc)):
            kv[("K", b, h)] = np.zeros((T, 128), np.float16)
            kv[("V", b, h)] = W.tokens(wl, "V", b, h, 0, T)
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, T, T, kv=kv)
    q = W.random_vectors(91, (B, len(alloc) * g, 128)).astype(np.float16)
    ref = attention.attend_cache(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, B, T, T, H.SCALE)
    rk, bits_k, rv, bits_v = zip(*alloc)
    for b in range(B):
        for h in range(len(alloc)):
            s0, s1, w = codec.record_slice(rv, bits_v, B, T, h, b, 0, T)
            vhat = codec.decode_records(cv_h[s0:s1].reshape(T, w), rv[h], bits_v[h]) @ bv[h].astype(np.float64).T
            mean = vhat.mean(axis=0)
            for i in range(g):
                assert np.abs(ref[b, h * g + i] - mean).max() <= 1e-9 * np.abs(mean).max()
    lay = K.Layout(len(alloc), len(alloc) * g, B, T, alloc)
    for split in (0, 256):
        got = _attend(K, lay, q, T, bk, bv, H.u32_dev(ck_h), H.u32_dev(cv_h), split)
        err = H.rel_err_per_head(got, ref)
        say(f"  split={split} max rel err {err:.3e}")
        assert err <= REL_TOL


def _near_basis_nullspace(P, n, seed, dtype):
    """Tokens almost orthogonal to the span of P: coordinates of the order of the
    float32 error bound, so that most header and code decisions are near a boundary
    at float32 precision (the exact float64 decisions are ordinary)."""
    rng = np.random.default_rng(seed)
    P = np.asarray(P, np.float64)
    z = rng.standard_normal((n, P.shape[0])) * 3.0
    x = z - (z @ P) @ P.T + (rng.standard_normal((n, P.shape[1])) * 1e-4) @ P.T
    return x.astype(np.float16 if dtype == "f16" else np.float32)


@pytest.mark.parametrize("dtype,scale", [("f16", 1.0), ("f32", 1.0), ("f16", 8.0), ("f32", 0.125)])
def test_prefill_records_equal_append_records(K, dtype, scale):
    """kv_encode (matrix-core projection, exact recomputation near rounding boundaries)
    writes the same records, bit for bit, as kv_append (float64 projection) token by
    token, for every rank and bit width, on ordinary tokens and on tokens whose
    coordinates sit within the float32 error bound of each other.  scale != 1: the
    bases are scaled (columns of norm 8 or 1/8, as a non-orthogonal key transform
    has), so the encoder's error bound must follow the basis' column norms."""
    say(f"prefill records == append records {dtype}, basis scale {scale}")
    wl = W.LLAMA_T32K
    alloc = MIXED_ALLOC
    hkv, B, n, pos0 = len(alloc), 2, 320, 5
    bk, bv = _mixed_bases(alloc, seed=11)
    lay = K.Layout(hkv, hkv, B, pos0 + n, alloc)
    tdt = torch.float32 if dtype == "f32" else torch.float16
    x = {}
    for t, bases in (("K", bk), ("V", bv)):
        x[t] = np.stack([np.stack([np.concatenate([W.tokens(wl, t, b, h, 0, n - 96, dtype),
                                                   _near_basis_nullspace(bases[h], 96, 100 * b + h, dtype)])
                                   for h in range(hkv)]) for b in range(B)])
    bk = [(p.astype(np.float64) * scale).astype(np.float32) for p in bk]
    bv = [(p.astype(np.float64) * scale).astype(np.float32) for p in bv]
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    kd, vd = H.dev(x["K"], tdt), H.dev(x["V"], tdt)
    nk, nv = K.kv_cache_bytes(lay, 0) // 4, K.kv_cache_bytes(lay, 1) // 4
    ck_e = torch.zeros(nk, dtype=torch.int32, device="cuda")
    cv_e = torch.zeros(nv, dtype=torch.int32, device="cuda")
    ck_a, cv_a = torch.zeros_like(ck_e), torch.zeros_like(cv_e)
    K.kv_encode(lay, kd, vd, n, pos0, pk, pv, ck_e, cv_e)
    for t in range(n):
        K.kv_append(lay, kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), pos0 + t, pk, pv, ck_a, cv_a)
    gk, gv = H.u32_host(ck_e), H.u32_host(cv_e)
    ak, av = H.u32_host(ck_a), H.u32_host(cv_a)
    assert np.array_equal(gk, ak), f"K records differ at {np.flatnonzero(gk != ak)[:8]}"
    assert np.array_equal(gv, av), f"V records differ at {np.flatnonzero(gv != av)[:8]}"
    rk, bits_k, rv, bits_v = zip(*alloc)
    for tensor, got_all, ranks, bits, bases in (("K", gk, rk, bits_k, bk), ("V", gv, rv, bits_v, bv)):
        for h in range(hkv):
            for b in range(B):
                s0, s1, w = codec.record_slice(ranks, bits, B, pos0 + n, h, b, pos0, pos0 + n)
                ref = codec.encode_tokens(x[tensor][b, h].astype(np.float64), bases[h], bits[h])
                H.compare_records(got_all[s0:s1].reshape(n, w), ref, ranks[h], bits[h], f"{tensor} h{h} b{b}",
                                 x[tensor][b, h], bases[h])


def test_append_matches_oracle(K):
    say("append mixed allocation")
    wl = W.QWEN_T128K
    alloc = [(128, 2, 128, 2), (16, 6, 16, 6)]
    bk, bv = _mixed_bases(alloc, seed=3)
    lay = _encode_case(K, lambda t, b, h, n: W.tokens(wl, t, b, h, 50, n), alloc, bk, bv, 3, 64, 63, 1, "f16")
    assert lay.capacity == 64


# ------------------------------------------------------------------ attention on an identical cache
def _attend(K, lay, q, T, bases_k, bases_v, ck, cv, split=0, qdtype=torch.float16):
    B, hq = lay.batch, lay.n_q_heads
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(K.kv_workspace_bytes(lay, T, split) // 4, dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q, qdtype), T, H.dev(codec.concat_bases(bases_k)),
                       H.dev(codec.concat_bases(bases_v)), ck, cv, H.SCALE, out, ws, split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _attention_case(K, alloc, bases_k, bases_v, batch, g, cap, T, splits, qdtype="f16", seed=0, wl=W.LLAMA_T32K):
    hkv = len(alloc)
    ck_h, cv_h = H.oracle_cache(wl, alloc, bases_k, bases_v, batch, cap, T,
                                kv={(t, b, h): W.tokens(wl, t, b, h % wl.n_kv_heads, 0, T)
                                    for t in "KV" for b in range(batch) for h in range(hkv)})
    q = W.random_vectors(seed, (batch, hkv * g, 128)).astype(np.float32 if qdtype == "f32" else np.float16)
    ref = attention.attend_cache(q.astype(np.float64), bases_k, bases_v, ck_h, cv_h, alloc, batch, cap, T, H.SCALE)
    lay = K.Layout(hkv, hkv * g, batch, cap, alloc)
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    errs = {}
    for split in splits:
        got = _attend(K, lay, q, T, bases_k, bases_v, ck, cv, split,
                      torch.float32 if qdtype == "f32" else torch.float16)
        assert np.isfinite(got).all()
        errs[split] = H.rel_err_per_head(got, ref)
        say(f"  split={split} max rel err {errs[split]:.3e}")
        assert errs[split] <= REL_TOL
    return errs


def test_attention_tiny_fp32(K):
    say("attention tiny-1head-T4096 fp32")
    wl = W.TINY
    alloc, bk, bv = H.oracle_calibrate(wl)
    _attention_case(K, alloc, bk, bv, 1, 1, 4096, 4096, [0, 256, 1024], qdtype="f32", wl=wl)


def test_attention_mixed_allocations_gqa4(K):
    say("attention mixed allocation g=4")
    bk, bv = _mixed_bases(MIXED_ALLOC, seed=5)
    _attention_case(K, MIXED_ALLOC, bk, bv, 2, 4, 3100, 3000, [0, 256, 768])


def test_attention_gqa7_qwen_allocation(K):
    say("attention g=7 (128,2)+(16,6)")
    alloc = [(128, 2, 128, 2), (16, 6, 16, 6)]
    bk, bv = _mixed_bases(alloc, seed=9)
    _attention_case(K, alloc, bk, bv, 2, 7, 2000, 1999, [0, 512], wl=W.QWEN_T128K)


def test_attention_every_bit_width(K):
    say("attention all bit widths")
    alloc = [(32, b, 64, 10 - b) for b in range(2, 9)]
    bk, bv = _mixed_bases(alloc, seed=13)
    _attention_case(K, alloc, bk, bv, 1, 2, 700, 700, [0, 256])


@pytest.mark.parametrize("T", [1, 2, 255, 256, 257])
def test_attention_short_and_ragged_contexts(K, T):
    say(f"attention T={T}")
    alloc = [(64, 4, 32, 8), (16, 8, 128, 2)]
    bk, bv = _mixed_bases(alloc, seed=17)
    _attention_case(K, alloc, bk, bv, 2, 3, T, T, [0])


@pytest.mark.parametrize("g", [1, 2, 3, 5, 8, 12])
def test_attention_group_sizes(K, g):
    """GQA groups below, at and above the specialised kernels' row blocks (4, 8; 12
    runs the generic kernel): query-head rows past g stay out of every sum."""
    say(f"attention g={g}")
    alloc = [(64, 4, 128, 2), (32, 8, 16, 8)]
    bk, bv = _mixed_bases(alloc, seed=41 + g)
    _attention_case(K, alloc, bk, bv, 2, g, 900, 873, [0, 256])


# The largest layouts the boundary accepts: 64 KV heads (the kernel-argument head
# table), and GQA groups of 16 query heads per KV head.
ALLOC_64_CLASS = [[(64, 4, 128, 2), (32, 8, 64, 4), (128, 2, 16, 8), (16, 8, 32, 8)][h % 4] for h in range(64)]
ALLOC_64_MIXED = [[(64, 4, 128, 2), (32, 3, 64, 5), (16, 6, 32, 7), (128, 4, 16, 2)][h % 4] for h in range(64)]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_encode_64_kv_heads(K, dtype):
    """Prefill encode of a 64-head layout (every head's own format) against the oracle."""
    say(f"encode 64 KV heads {dtype}")
    wl = W.LLAMA_T32K
    bk, bv = _mixed_bases(ALLOC_64_MIXED, seed=71)
    _encode_case(K, lambda t, b, h, n: W.tokens(wl, t, b, h % wl.n_kv_heads, 0, n, dtype), ALLOC_64_MIXED, bk, bv,
                 1, 200, 3, 150, dtype)


@pytest.mark.parametrize("alloc", [ALLOC_64_CLASS, ALLOC_64_MIXED], ids=["class-kernel", "generic-kernel"])
def test_attention_64_kv_heads(K, alloc):
    """Decode attention over 64 KV heads (GQA group 2), on the class kernel and on the
    generic one."""
    say(f"attention 64 KV heads, class {K.kv_attend_plan(K.Layout(64, 128, 1, 300, alloc), 300)[0]}")
    bk, bv = _mixed_bases(alloc, seed=73)
    _attention_case(K, alloc, bk, bv, 1, 2, 300, 300, [0, 256])


def test_attention_group_16(K):
    """The largest GQA group: 16 query heads per KV head (two value operands per row
    block, the generic kernel), with several splits."""
    say("attention g=16")
    alloc = [(64, 4, 128, 2), (32, 5, 16, 8)]
    bk, bv = _mixed_bases(alloc, seed=79)
    _attention_case(K, alloc, bk, bv, 2, 16, 900, 873, [0, 256])


def _budget_formats(budget_bits):
    """(rank, bits) the per-head search can pick under one budget of bits per vector:
    b = min(8, floor(budget / r)) for every rank with b >= 2."""
    return [(r, min(8, budget_bits // r)) for r in (16, 32, 64, 128) if min(8, budget_bits // r) >= 2]


@pytest.mark.parametrize("budget", [64, 128, 256, 512])
@pytest.mark.parametrize("g", [4, 7])
def test_attention_every_format_pair_of_a_budget(K, budget, g):
    """All (K, V) format pairs of one budget in one layout (the specialised kernels)."""
    fm = _budget_formats(budget)
    alloc = [(rk, bk, rv, bv) for (rk, bk) in fm for (rv, bv) in fm]
    say(f"attention budget {budget} bits, g={g}, {len(alloc)} heads")
    bk, bv = _mixed_bases(alloc, seed=31 + budget + g)
    _attention_case(K, alloc, bk, bv, 1, g, 800, 777, [0, 256])


# the frozen cross-head (C2) allocation of the LLaMA-shaped layer at 2 bits/dim (odd widths)
C2_LLAMA_2BPD = [(64, 4, 128, 3), (128, 4, 128, 3), (32, 5, 16, 5), (128, 3, 16, 5),
                 (128, 4, 32, 4), (16, 4, 128, 3), (16, 5, 128, 4), (16, 5, 32, 3)]


@pytest.mark.parametrize("g", [4, 7])
def test_attention_frozen_cross_head_allocation(K, g):
    """The eight per-head format pairs of a frozen C2 allocation in one layout."""
    say(f"attention C2 allocation, g={g}")
    bk, bv = _mixed_bases(C2_LLAMA_2BPD, seed=61 + g)
    _attention_case(K, C2_LLAMA_2BPD, bk, bv, 2, g, 1100, 1037, [0, 256])


def test_attention_ragged_lengths(K):
    """kv_attend_decode_ragged: each sequence against the oracle over its own tokens
    (a zero length gives zeros, a length past max_tokens is clamped to it), and with
    every length equal to max_tokens the output equals kv_attend_decode's bit for bit."""
    alloc = [(64, 4, 32, 8), (16, 6, 128, 3)]
    bk, bv = _mixed_bases(alloc, seed=71)
    batch, g, cap, T = 4, 4, 3200, 3100
    lens = [1000, 0, 257, 5000]
    say(f"attention ragged lengths {lens}, max {T}")
    hkv, wl = len(alloc), W.LLAMA_T32K
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, batch, cap, T,
                                kv={(t, b, h): W.tokens(wl, t, b, h, 0, T)
                                    for t in "KV" for b in range(batch) for h in range(hkv)})
    q = W.random_vectors(3, (batch, hkv * g, 128)).astype(np.float16)
    lay = K.Layout(hkv, hkv * g, batch, cap, alloc)
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    out = torch.full((batch, hkv * g, 128), float("nan"), dtype=torch.float32, device="cuda")
    qd = H.dev(q, torch.float16)
    K.kv_attend_decode_ragged(lay, qd, torch.tensor(lens, dtype=torch.int32, device="cuda"), T, pk, pv, ck, cv,
                              H.SCALE, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, lb in enumerate(lens):
        tb = min(max(lb, 0), T)
        if tb == 0:
            assert (got[b] == 0).all()
            continue
        ref = attention.attend_cache(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, batch, cap, tb, H.SCALE)
        err = H.rel_err_per_head(got[b:b + 1], ref[b:b + 1])
        say(f"  sequence {b} length {tb}: max rel err {err:.3e}")
        assert err <= REL_TOL
    K.kv_attend_decode_ragged(lay, qd, torch.full((batch,), T, dtype=torch.int32, device="cuda"), T, pk, pv, ck, cv,
                              H.SCALE, out, ws)
    torch.cuda.synchronize()
    same = _attend(K, lay, q, T, bk, bv, ck, cv)
    assert np.array_equal(out.cpu().numpy(), same)


def test_attention_workspace_reuse_across_calls(K):
    """One zero-filled workspace serves consecutive calls with different split counts:
    every call leaves its split arrival counters at zero for the next."""
    say("attention: one workspace, several calls")
    wl = W.LLAMA_T32K
    alloc = [(64, 4, 64, 4), (128, 2, 32, 8)]
    bk, bv = _mixed_bases(alloc, seed=23)
    B, g, T = 2, 4, 1500
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, T, T,
                                kv={(t, b, h): W.tokens(wl, t, b, h, 0, T) for t in "KV" for b in range(B) for h in range(2)})
    q = W.random_vectors(29, (B, 2 * g, 128)).astype(np.float16)
    ref = attention.attend_cache(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, B, T, T, H.SCALE)
    lay = K.Layout(2, 2 * g, B, T, alloc)
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    splits = [256, 0, 512, 256, 1536]
    ws = torch.zeros(max(K.kv_workspace_bytes(lay, T, s) for s in splits) // 4, dtype=torch.float32, device="cuda")
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    qd = H.dev(q, torch.float16)
    for split in splits:
        out = torch.empty((B, 2 * g, 128), dtype=torch.float32, device="cuda")
        K.kv_attend_decode(lay, qd, T, pk, pv, ck, cv, H.SCALE, out, ws, split_tokens=split)
        torch.cuda.synchronize()
        err = H.rel_err_per_head(out.cpu().numpy(), ref)
        say(f"  split={split} max rel err {err:.3e}")
        assert err <= REL_TOL
    cnt = ws[: 2 * B].view(torch.int32).cpu().numpy()
    assert (cnt == 0).all()


def _n_splits(K, lay, T, split=0):
    """Largest per-head split count of a launch, read back from its workspace size."""
    units = lay.batch * lay.n_kv_heads
    words = K.kv_workspace_bytes(lay, T, split) // 4 - (units + 3) // 4 * 4
    return words // (lay.batch * lay.n_q_heads * 132)


@pytest.mark.parametrize("g", [2, 4, 8])
def test_attention_more_than_32_splits(K, g):
    """66 splits per (sequence, KV head): the split merge's multi-round path (two
    threads per output quad for g <= 4, each folding three rounds of up to 16
    splits and then exchanging; one thread and five rounds for g = 8)."""
    alloc = [(64, 4, 32, 8), (32, 8, 64, 4)]
    bk, bv = _mixed_bases(alloc, seed=83 + g)
    T = 16700
    lay = K.Layout(len(alloc), len(alloc) * g, 1, T, alloc)
    ns = _n_splits(K, lay, T, 256)
    say(f"attention g={g}, T={T}, split 256: {ns} splits per unit")
    assert ns > 32
    _attention_case(K, alloc, bk, bv, 1, g, T, T, [256, 0])


def test_attention_dirty_workspace_is_nan_or_correct(K):
    """Split arrival counters that are not zero on entry (above, at and below the
    split count, and an all-ones word) and stale partials: every output element is
    NaN or bit-equal to the output of a zero-filled workspace, on this call and the
    next; a zero-filled workspace afterwards gives the exact output again, and the
    kernel exits normally throughout."""
    alloc = [(64, 4, 64, 4), (128, 2, 32, 8)]
    bk, bv = _mixed_bases(alloc, seed=89)
    B, g, T, split = 2, 4, 3000, 256
    hkv = len(alloc)
    wl = W.LLAMA_T32K
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, T, T,
                                kv={(t, b, h): W.tokens(wl, t, b, h, 0, T) for t in "KV" for b in range(B)
                                    for h in range(hkv)})
    q = W.random_vectors(97, (B, hkv * g, 128)).astype(np.float16)
    lay = K.Layout(hkv, hkv * g, B, T, alloc)
    ns = _n_splits(K, lay, T, split)
    say(f"dirty workspace: {ns} splits per unit")
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    qd = H.dev(q, torch.float16)
    nw = K.kv_workspace_bytes(lay, T, split) // 4
    clean = torch.zeros(nw, dtype=torch.float32, device="cuda")
    ref = torch.empty((B, hkv * g, 128), dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, qd, T, pk, pv, ck, cv, H.SCALE, ref, clean, split_tokens=split)
    torch.cuda.synchronize()
    assert (clean[: B * hkv].view(torch.int32) == 0).all()
    oracle = attention.attend_cache(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, B, T, T, H.SCALE)
    assert H.rel_err_per_head(ref.cpu().numpy(), oracle) <= REL_TOL
    ref_bits = ref.cpu().numpy().view(np.uint32)
    # partials left by the clean call (another call's tags), counters preset
    dirty = clean.clone()
    cnt = np.array([0xFFFFFFFF, ns + 7, ns, ns - 1], np.uint32)[: B * hkv]
    dirty[: B * hkv] = torch.from_numpy(cnt.view(np.int32)).cuda().view(torch.float32)
    n_nan = 0
    for rep in range(2):
        out = torch.full_like(ref, 7.0)
        K.kv_attend_decode(lay, qd, T, pk, pv, ck, cv, H.SCALE, out, dirty, split_tokens=split)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        nan = np.isnan(got)
        same = got.view(np.uint32) == ref_bits
        assert (nan | same).all(), f"call {rep}: {(~(nan | same)).sum()} elements neither NaN nor correct"
        n_nan += int(nan.sum())
        say(f"  call {rep}: {int(nan.sum())} NaN elements, the rest exact; counters "
            f"{dirty[: B * hkv].view(torch.int32).cpu().numpy().view(np.uint32).tolist()}")
    dirty.zero_()
    out = torch.empty_like(ref)
    K.kv_attend_decode(lay, qd, T, pk, pv, ck, cv, H.SCALE, out, dirty, split_tokens=split)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref_bits)


def test_full_size_llama_b1_t32k_fused_step(K):
    """The LLaMA-shaped single-sequence layer at its own size: 32 query heads over 8 KV
    heads, C1 at 2 bits per dimension with MSE weights, a 32768-token prefill encoded
    on the GPU, then one decode step (the append of token 32768 fused with attention
    over all 32769 tokens) with the default split plan (32 splits per unit, at most
    T / 1024: the merge folds them in one round).
    The fused step equals kv_append + kv_attend_decode bit for bit; every unit's
    records match the oracle's (exact headers, codes only at classified ties) and all
    32 query heads' outputs match oracle attention."""
    wl = W.LLAMA_T32K
    T = wl.context + 1
    B, hkv, hq, g = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.group
    alloc, bk, bv = H.oracle_calibrate(wl)
    lay = K.Layout(hkv, hq, B, T, alloc)
    ns = _n_splits(K, lay, T)
    say(f"full size {wl.name}: {alloc}, {ns} splits per unit")
    assert ns == 32
    kx = W.kv_array(wl, "K", 0, T)
    vx = W.kv_array(wl, "V", 0, T)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    K.kv_encode(lay, H.dev(kx[:, :, :T - 1]), H.dev(vx[:, :, :T - 1]), T - 1, 0, pk, pv, ck, cv)
    k1, v1 = H.dev(kx[:, :, T - 1]), H.dev(vx[:, :, T - 1])
    q = W.query_array(wl, 0)
    qd = H.dev(q)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    ck2, cv2 = ck.clone(), cv.clone()
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    K.kv_append_attend_decode(lay, k1, v1, qd, T, pk, pv, ck, cv, H.SCALE, out, ws)
    out2 = torch.empty_like(out)
    K.kv_append(lay, k1, v1, T - 1, pk, pv, ck2, cv2)
    K.kv_attend_decode(lay, qd, T, pk, pv, ck2, cv2, H.SCALE, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(ck, ck2) and torch.equal(cv, cv2), "fused append wrote other records"
    assert torch.equal(out, out2), "fused step differs from append + attend"
    assert (ws[: B * hkv].view(torch.int32) == 0).all()
    got = out.cpu().numpy()
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bits_k, rv, bits_v = zip(*alloc)
    worst = 0.0
    for h in range(hkv):
        rec_k = codec.encode_tokens(kx[0, h], bk[h], bits_k[h])
        rec_v = codec.encode_tokens(vx[0, h], bv[h], bits_v[h])
        s0, s1, w = codec.record_slice(rk, bits_k, B, T, h, 0, 0, T)
        H.compare_records(gk[s0:s1].reshape(-1, w), rec_k, rk[h], bits_k[h], f"K h{h}", kx[0, h], bk[h])
        s0, s1, w = codec.record_slice(rv, bits_v, B, T, h, 0, 0, T)
        H.compare_records(gv[s0:s1].reshape(-1, w), rec_v, rv[h], bits_v[h], f"V h{h}", vx[0, h], bv[h])
        ref = attention.attend_head_records(q[0, h * g:(h + 1) * g].astype(np.float64), bk[h], rec_k, rk[h],
                                            bits_k[h], bv[h], rec_v, rv[h], bits_v[h], H.SCALE)
        err = H.rel_err_per_head(got[0, h * g:(h + 1) * g], ref)
        worst = max(worst, err)
        assert err <= REL_TOL, f"KV head {h}: max rel err {err:.3e}"
    say(f"  all 8 units: records match, max rel err {worst:.3e}")


# ------------------------------------------------------------------ append fused with attention
FUSED_CASES = [
    # allocation, query heads per KV head, batch, capacity, tokens after the append, split, k1/v1 dtype
    pytest.param([(128, 2, 128, 2), (64, 4, 32, 8)], 4, 2, 600, 1, 0, "f16", id="first-token"),
    pytest.param([(128, 2, 128, 2), (64, 4, 32, 8)], 4, 2, 600, 256, 256, "f16", id="last-of-split"),
    pytest.param([(128, 2, 128, 2), (64, 4, 32, 8)], 4, 2, 600, 257, 256, "f32", id="first-of-split"),
    pytest.param(MIXED_ALLOC, 4, 2, 1600, 1500, 0, "f32", id="mixed-ragged"),
    pytest.param([(32, 3, 64, 5), (16, 7, 128, 6)], 7, 1, 800, 777, 256, "f16", id="odd-widths-g7"),
    pytest.param([(64, 4, 64, 4), (16, 8, 128, 4)], 8, 1, 600, 513, 512, "f16", id="g8"),
    pytest.param([(64, 4, 128, 2), (32, 5, 16, 8)], 16, 1, 700, 650, 256, "f16", id="g16-largest-group"),
]


@pytest.mark.parametrize("alloc,g,B,cap,T,split,kvdt", FUSED_CASES)
def test_fused_append_attend(K, alloc, g, B, cap, T, split, kvdt):
    """kv_append_attend_decode against kv_append + kv_attend_decode on copies of one
    cache (records and output bit-identical), and against the oracle (the new
    record up to rounding ties, the output within the attention tolerance)."""
    say(f"fused append+attend T={T} split={split} g={g} {kvdt}")
    wl = W.LLAMA_T32K
    hkv = len(alloc)
    bk, bv = _mixed_bases(alloc, seed=41 + T)
    kv = {(t, b, h): W.tokens(wl, t, b, h, 0, T, kvdt) for t in "KV" for b in range(B) for h in range(hkv)}
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T - 1, kv={key: x[: T - 1] for key, x in kv.items()})
    lay = K.Layout(hkv, hkv * g, B, cap, alloc)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    tdt = torch.float32 if kvdt == "f32" else torch.float16
    k1 = H.dev(np.stack([np.stack([kv["K", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), tdt)
    v1 = H.dev(np.stack([np.stack([kv["V", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), tdt)
    q = H.dev(W.random_vectors(43 + T, (B, hkv * g, 128)).astype(np.float16), torch.float16)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T, split) // 4, dtype=torch.float32, device="cuda")

    ck_f, cv_f = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_f = torch.full((B, hkv * g, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kv_append_attend_decode(lay, k1, v1, q, T, pk, pv, ck_f, cv_f, H.SCALE, out_f, ws, split_tokens=split)
    ck_s, cv_s = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_s = torch.full_like(out_f, float("nan"))
    K.kv_append(lay, k1, v1, T - 1, pk, pv, ck_s, cv_s)
    K.kv_attend_decode(lay, q, T, pk, pv, ck_s, cv_s, H.SCALE, out_s, ws, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(ck_f, ck_s) and torch.equal(cv_f, cv_s), "fused append wrote other records"
    assert torch.equal(out_f, out_s), "fused output differs from append + attend"
    assert (ws[: hkv * B].view(torch.int32) == 0).all()

    ok_h, ov_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T, kv=kv)
    gk, gv = H.u32_host(ck_f), H.u32_host(cv_f)
    rk, bits_k, rv, bits_v = zip(*alloc)
    for h in range(hkv):
        for b in range(B):
            for got, ref, ranks, bits, name, bases in ((gk, ok_h, rk, bits_k, "K", bk), (gv, ov_h, rv, bits_v, "V", bv)):
                s0, s1, w = codec.record_slice(ranks, bits, B, cap, h, b, 0, T)
                H.compare_records(got[s0:s1].reshape(T, w), ref[s0:s1].reshape(T, w), ranks[h], bits[h],
                                 f"{name} h{h} b{b}", kv[name, b, h], bases[h])
    ref = attention.attend_cache(q.cpu().numpy().astype(np.float64), bk, bv, ok_h, ov_h, alloc, B, cap, T, H.SCALE)
    err = H.rel_err_per_head(out_f.cpu().numpy(), ref)
    say(f"  max rel err {err:.3e}")
    assert err <= REL_TOL


@pytest.mark.parametrize("alloc", [MIXED_ALLOC, [(64, 4, 128, 2), (32, 8, 64, 4)]], ids=["generic", "specialised"])
def test_attention_repeatable_bit_for_bit(K, alloc):
    """The fixed split boundaries, tile-to-wave assignment and summation orders make
    the output a function of the inputs alone: repeated calls, and calls on a copy
    of the cache at another address, give the same bits."""
    say(f"attention: repeated calls are bit-identical {alloc}")
    wl = W.LLAMA_T32K
    bk, bv = _mixed_bases(alloc, seed=53)
    B, g, T = 2, 4, 5000
    hkv = len(alloc)
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, T, T,
                                kv={(t, b, h): W.tokens(wl, t, b, h % wl.n_kv_heads, 0, T)
                                    for t in "KV" for b in range(B) for h in range(hkv)})
    q = W.random_vectors(59, (B, hkv * g, 128)).astype(np.float16)
    lay = K.Layout(hkv, hkv * g, B, T, alloc)
    ck, cv = H.u32_dev(ck_h), H.u32_dev(cv_h)
    outs = [_attend(K, lay, q, T, bk, bv, ck, cv) for _ in range(3)]
    ck2, cv2 = ck.clone(), cv.clone()
    outs.append(_attend(K, lay, q, T, bk, bv, ck2, cv2))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    ref = attention.attend_cache(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, B, T, T, H.SCALE)
    assert H.rel_err_per_head(outs[0], ref) <= REL_TOL


def test_attention_empty_context_is_zero(K):
    say("attention T=0")
    alloc = [(64, 4, 32, 8)]
    bk, bv = _mixed_bases(alloc, seed=19)
    lay = K.Layout(1, 2, 1, 16, alloc)
    ck = H.u32_dev(np.zeros(K.kv_cache_bytes(lay, 0) // 4, np.uint32))
    cv = H.u32_dev(np.zeros(K.kv_cache_bytes(lay, 1) // 4, np.uint32))
    got = _attend(K, lay, W.random_vectors(1, (1, 2, 128)).astype(np.float16), 0, bk, bv, ck, cv)
    assert np.array_equal(got, np.zeros_like(got))


# ------------------------------------------------------------------ end to end
def test_end_to_end_encode_append_attend(K):
    say("end to end: encode + append + attend")
    wl = W.LLAMA_T32K
    alloc, bk, bv = H.oracle_calibrate(wl)
    B, T = 1, 2000
    lay = K.Layout(wl.n_kv_heads, wl.n_q_heads, B, T + 1, alloc)
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    kx = np.stack([np.stack([W.tokens(wl, "K", b, h, 0, T + 1) for h in range(wl.n_kv_heads)]) for b in range(B)])
    vx = np.stack([np.stack([W.tokens(wl, "V", b, h, 0, T + 1) for h in range(wl.n_kv_heads)]) for b in range(B)])
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    K.kv_encode(lay, H.dev(kx[:, :, :T]), H.dev(vx[:, :, :T]), T, 0, pk, pv, ck, cv)
    K.kv_append(lay, H.dev(kx[:, :, T]), H.dev(vx[:, :, T]), T, pk, pv, ck, cv)
    q = W.query_array(wl, 0)
    got = _attend(K, lay, q, T + 1, bk, bv, ck, cv)
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, T + 1, T + 1,
                                kv={(t, b, h): (kx if t == "K" else vx)[b, h]
                                    for t in "KV" for b in range(B) for h in range(wl.n_kv_heads)})
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bits_k, rv, bits_v = zip(*alloc)
    for h in range(wl.n_kv_heads):
        s0, s1, w = codec.record_slice(rk, bits_k, B, T + 1, h, 0, 0, T + 1)
        H.compare_records(gk[s0:s1].reshape(-1, w), ck_h[s0:s1].reshape(-1, w), rk[h], bits_k[h], f"K h{h}",
                         kx[0, h], bk[h])
        s0, s1, w = codec.record_slice(rv, bits_v, B, T + 1, h, 0, 0, T + 1)
        H.compare_records(gv[s0:s1].reshape(-1, w), cv_h[s0:s1].reshape(-1, w), rv[h], bits_v[h], f"V h{h}",
                         vx[0, h], bv[h])
    ref = attention.attend_cache(q.astype(np.float64), bk, bv, ck_h, cv_h, alloc, B, T + 1, T + 1, H.SCALE)
    err = H.rel_err_per_head(got, ref)
    say(f"  end-to-end max rel err {err:.3e}")
    assert err <= REL_TOL


# ------------------------------------------------------------------ full size, sampled
FULL_SIZE = {"llama-2bpd": lambda: W.llama_t128k(2.0), "llama-0.5bpd": lambda: W.llama_t128k(0.5),
             "llama-1bpd": lambda: W.llama_t128k(1.0), "llama-4bpd": lambda: W.llama_t128k(4.0),
             "qwen-mixed": lambda: W.QWEN_T128K,
             "llama-B16-T32K-r32b8": lambda: W.llama_prefill(32, 8),
             "llama-B16-T32K-r64b4": lambda: W.llama_prefill(64, 4),
             "llama-2bpd-c2": lambda: W.llama_t128k_c2(2.0)}


@pytest.mark.parametrize("name", list(FULL_SIZE))
def test_full_size_128k_sampled_units(K, name):
    """The decode configurations at full size (LLaMA shape at 128K: 4 sequences x 8 KV
    heads at 0.5, 1, 2 and 4 bits per dimension; Qwen shape: 8 sequences x 4 KV heads;
    both with 131073 tokens; LLaMA shape at 32K: 16 sequences x 8 KV heads, 32769
    tokens, uniform r = 32 b = 8 or r = 64 b = 4), encoded on the GPU and attended
    with the default split, in the launch configuration the benchmark times.  Sampled
    (sequence, KV head) units are re-encoded by the oracle from the same inputs: their
    records must match (exact headers, codes off by one only at rounding ties) and their
    query heads' outputs are checked against oracle attention."""
    wl = FULL_SIZE[name]()
    T = wl.context + 1
    B, hkv, hq, d, g = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.group
    alloc, bk, bv = H.oracle_calibrate(wl)
    say(f"full size {wl.name}: {alloc}")
    lay = K.Layout(hkv, hq, B, T, alloc)
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device="cuda")
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device="cuda")
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    for t0 in range(0, T, 1 << 15):
        n = min(1 << 15, T - t0)
        K.kv_encode(lay, H.dev(W.kv_array(wl, "K", t0, n)), H.dev(W.kv_array(wl, "V", t0, n)), n, t0, pk, pv, ck, cv)
    q = W.query_array(wl, 0)
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device="cuda")
    K.kv_attend_decode(lay, H.dev(q), T, pk, pv, ck, cv, H.SCALE, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gk, gv = H.u32_host(ck), H.u32_host(cv)
    rk, bits_k, rv, bits_v = zip(*alloc)
    for b, h in [(0, 0), (B - 1, hkv - 1), (1, hkv // 2)]:
        xk = W.tokens(wl, "K", b, h, 0, T)
        xv = W.tokens(wl, "V", b, h, 0, T)
        rec_k = np.concatenate([codec.encode_tokens(xk[i:i + 16384], bk[h], bits_k[h]) for i in range(0, T, 16384)])
        rec_v = np.concatenate([codec.encode_tokens(xv[i:i + 16384], bv[h], bits_v[h]) for i in range(0, T, 16384)])
        s0, s1, w = codec.record_slice(rk, bits_k, B, T, h, b, 0, T)
        fk = H.compare_records(gk[s0:s1].reshape(-1, w), rec_k, rk[h], bits_k[h], f"K b{b} h{h}", xk, bk[h])
        s0, s1, w = codec.record_slice(rv, bits_v, B, T, h, b, 0, T)
        fv = H.compare_records(gv[s0:s1].reshape(-1, w), rec_v, rv[h], bits_v[h], f"V b{b} h{h}", xv, bv[h])
        ref = attention.attend_head_records(q[b, h * g:(h + 1) * g].astype(np.float64), bk[h], rec_k, rk[h], bits_k[h],
                                            bv[h], rec_v, rv[h], bits_v[h], H.SCALE)
        err = H.rel_err_per_head(got[b, h * g:(h + 1) * g], ref)
        say(f"  unit (b={b}, h={h}) {alloc[h]}: code mismatch K {fk:.1e} V {fv:.1e}, max rel err {err:.3e}")
        assert err <= REL_TOL
