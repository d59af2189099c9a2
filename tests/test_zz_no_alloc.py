"""kv_append_attend_decode_noalloc (split scratch in the library's static device
array) against kv_append_attend_decode (the caller's workspace): the same records
and bit-identical outputs, on two calls in a row (the second with a smaller
layout, batch and context), and against oracle attention; requests larger than
the static scratch are refused before anything is launched."""
import numpy as np
import pytest

import harness as H
import workloads as W
from oracle import attention, codec, transform

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_04_amd as K
    K.kv_record_words(16, 2)
    return K


def _bases(alloc, seed):
    bk, bv = [], []
    for h, (rk, _, rv, _) in enumerate(alloc):
        bk.append(transform.basis_for_head(W.random_covariance(seed + h, 128), rk,
                                           W.random_basis_signs(seed + 20 + h, rk)).astype(np.float32))
        bv.append(transform.basis_for_head(W.random_covariance(seed + 40 + h, 128), rv,
                                           W.random_basis_signs(seed + 60 + h, rv)).astype(np.float32))
    return bk, bv


def _step_both_ways(K, alloc, g, B, cap, T, split, seed):
    wl = W.LLAMA_T32K
    hkv = len(alloc)
    bk, bv = _bases(alloc, seed)
    kv = {(t, b, h): W.tokens(wl, t, b, h, 0, T) for t in "KV" for b in range(B) for h in range(hkv)}
    ck_h, cv_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T - 1, kv={k: x[: T - 1] for k, x in kv.items()})
    lay = K.Layout(hkv, hkv * g, B, cap, alloc)
    pk, pv = H.dev(codec.concat_bases(bk)), H.dev(codec.concat_bases(bv))
    k1 = H.dev(np.stack([np.stack([kv["K", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), torch.float16)
    v1 = H.dev(np.stack([np.stack([kv["V", b, h][T - 1] for h in range(hkv)]) for b in range(B)]), torch.float16)
    q = H.dev(W.random_vectors(seed + 7, (B, hkv * g, 128)).astype(np.float16), torch.float16)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T, split) // 4, dtype=torch.float32, device="cuda")
    ck_w, cv_w = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_w = torch.full((B, hkv * g, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kv_append_attend_decode(lay, k1, v1, q, T, pk, pv, ck_w, cv_w, H.SCALE, out_w, ws, split_tokens=split)
    ck_s, cv_s = H.u32_dev(ck_h), H.u32_dev(cv_h)
    out_s = torch.full_like(out_w, float("nan"))
    K.kv_append_attend_decode_noalloc(lay, k1, v1, q, T, pk, pv, ck_s, cv_s, H.SCALE, out_s, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(ck_w, ck_s) and torch.equal(cv_w, cv_s), "records differ"
    assert torch.equal(out_w, out_s), "output differs from the workspace entry point's"
    ok_h, ov_h = H.oracle_cache(wl, alloc, bk, bv, B, cap, T, kv=kv)
    ref = attention.attend_cache(q.cpu().numpy().astype(np.float64), bk, bv, ok_h, ov_h, alloc, B, cap, T, H.SCALE)
    err = H.rel_err_per_head(out_s.cpu().numpy(), ref)
    print(f"noalloc step B={B} g={g} T={T} split={split}: bit-equal to the workspace call, "
          f"max rel err {err:.3e}", flush=True)
    assert err <= 2e-3


def test_noalloc_matches_workspace_entry_point_twice(K):
    # a larger call first, then a smaller layout, batch and context on the same static scratch
    _step_both_ways(K, [(64, 4, 128, 2), (32, 5, 64, 4), (128, 2, 16, 6)], 4, 3, 2600, 2500, 0, 101)
    _step_both_ways(K, [(16, 8, 32, 8)], 2, 1, 800, 700, 256, 131)


def test_noalloc_refuses_requests_beyond_the_static_scratch(K):
    lay = K.Layout(8, 128, 32, 9000, [(64, 4, 64, 4)] * 8)
    t = torch.zeros(16, dtype=torch.float16, device="cuda")
    with pytest.raises(K.KvError) as e:
        K.kv_append_attend_decode_noalloc(lay, t, t, t, 8192, t, t, t, t, H.SCALE, t, split_tokens=256)
    assert e.value.status == K.KV_ERR_CAPACITY
    assert "static scratch" in str(e.value)
