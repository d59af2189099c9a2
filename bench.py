"""Decode-attention throughput over the transform-coded KV cache on one MI355X.

One step = one decode step of one layer at 128K context, one launch of
kv_append_attend_decode: the append of the new token's key and value (encode:
project -> quantize -> pack) and the attention over the T+1 compressed records
of every (sequence, KV head) (query projection, split-K attention over packed
codes, log-sum-exp combine and value back-projection).  Before timing, the same
step as two calls (kv_append, then kv_attend_decode) must give a bit-identical
output.  Inputs are resident in HBM before timing starts;
steps rotate over several layer caches (>= 1 GB in total) so that no step is
served from the 256 MB Infinity Cache.

Prints one JSON line (metric, value, roofline, cpu_baseline, ...); details go to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn compressed-KV GB/s (% of HBM peak) + context tokens/s @128K"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pick_workload(name: str) -> W.Workload:
    table = {
        "tiny": W.TINY,
        "llama-32k": W.LLAMA_T32K,
        "qwen-128k": W.QWEN_T128K,
        "llama-prefill-r32b8": W.llama_prefill(32, 8),
        "llama-prefill-r64b4": W.llama_prefill(64, 4),
    }
    for bpd in W.ALL_BUDGETS:
        table[f"llama-128k-{bpd:g}bpd"] = W.llama_t128k(bpd)
        table[f"llama-128k-{bpd:g}bpd-c2"] = W.llama_t128k_c2(bpd)
    if name not in table:
        raise SystemExit(f"unknown workload {name}; choose from {sorted(table)}")
    return table[name]


def calibrate(wl: W.Workload):
    """(allocation, key bases, value bases) of every KV head; with the attention-aware key
    transform each key entry is the head's flat [P_K; Q_K] block."""
    from decode_attention_04_amd import calib

    if wl.allocation[0] == "nova":
        out = [calib.calibrate_head_nova(W.covariance(wl, "K", h), W.covariance(wl, "V", h), W.query_covariance(wl, h),
                                         lambda r, h=h: W.hadamard_signs(wl, "K", h, r),
                                         lambda r, h=h: W.hadamard_signs(wl, "V", h, r), wl.allocation[1],
                                         head_dim=wl.head_dim) for h in range(wl.n_kv_heads)]
        return [o[0] for o in out], [o[1] for o in out], [o[2] for o in out]

    if wl.allocation[0] == "c2":
        n = wl.n_kv_heads
        return calib.calibrate_layer(
            [W.covariance(wl, "K", h) for h in range(n)], [W.covariance(wl, "V", h) for h in range(n)],
            lambda h, r: W.hadamard_signs(wl, "K", h, r), lambda h, r: W.hadamard_signs(wl, "V", h, r),
            wl.allocation, [W.query_covariance(wl, h) for h in range(n)], head_dim=wl.head_dim)
    alloc, bk, bv = [], [], []
    for h in range(wl.n_kv_heads):
        fixed = wl.allocation[1][h] if wl.allocation[0] == "fixed" else None
        a, pk, pv = calib.calibrate_head(
            W.covariance(wl, "K", h), W.covariance(wl, "V", h),
            lambda r, h=h: W.hadamard_signs(wl, "K", h, r), lambda r, h=h: W.hadamard_signs(wl, "V", h, r),
            wl.allocation, W.query_covariance(wl, h), fixed=fixed, head_dim=wl.head_dim)
        alloc.append(a)
        bk.append(pk)
        bv.append(pv)
    return alloc, bk, bv


def calibrate_vq(wl: W.Workload):
    """(allocation, key blocks [P_K; Q_K], value bases, K codebook words, V codebook words) of
    a workload with vector-quantized pairs, from the product's calibration: codebooks
    fitted on the training sequence's tokens (disjoint from the measured ones)."""
    from decode_attention_04_amd import calib

    bits = wl.allocation[1]
    m, kcw = wl.head_dim // 2, 1 << bits
    out = []
    for h in range(wl.n_kv_heads):
        xk = W.tokens(wl, "K", W.VQ_TRAIN_SEQ, h, 0, W.VQ_TRAIN_TOKENS).astype(np.float64)
        xv = W.tokens(wl, "V", W.VQ_TRAIN_SEQ, h, 0, W.VQ_TRAIN_TOKENS).astype(np.float64)
        out.append(calib.calibrate_head_nova_vq(
            W.covariance(wl, "K", h), W.covariance(wl, "V", h), W.query_covariance(wl, h), xk, xv, bits,
            W.vq_starts(wl, "K", h, m, kcw), W.vq_starts(wl, "V", h, m, kcw), W.VQ_ITERS))
    return tuple([o[i] for o in out] for i in range(5))


def step_bytes(wl, alloc, T, static=False):
    """Algorithmic HBM bytes of one decode step: attention part and append part
    (static: header-free records, one word fewer each; vector-quantized pairs: the
    scale word and r/2 indices per record, plus the codebooks once)."""
    from decode_attention_04_amd import kv_record_words

    B, hq, d = wl.batch, wl.n_q_heads, wl.head_dim
    esz = 4 if wl.dtype == "f32" else 2
    vq = wl.allocation[0] == "nova-vq"
    if vq:
        rec = sum(4 * (2 + (a[0] // 2 * a[1] + 31) // 32 + (a[2] // 2 * a[3] + 31) // 32) for a in alloc)
        tables = sum(4 * ((a[0] // 2 << a[1]) + (a[2] // 2 << a[3])) for a in alloc)
    else:
        rec = sum(4 * (kv_record_words(a[0], a[1]) + kv_record_words(a[2], a[3]) - (2 if static else 0))
                  for a in alloc)
        tables = 0
    nk = 2 if wl.allocation[0] in ("nova", "nova-vq") else 1  # the attention-aware transform reads P_K and Q_K
    basis = sum(4 * d * (nk * a[0] + a[2]) for a in alloc) + tables
    attend = B * T * rec + B * hq * d * esz + basis + B * hq * d * 4
    append = B * wl.n_kv_heads * 2 * d * esz + B * rec + basis
    return attend, append


def encode_rate(K, wl, block=2048, reps=5):
    """kv_encode of the workload's prefill chunk (every sequence and KV head at once).

    Inputs: the workload's generated keys and values for the first `block` tokens,
    repeated along the token axis to the chunk length on the GPU (same per-token
    statistics, so the same share of coordinates near a rounding boundary)."""
    import torch

    dev = torch.device("cuda:0")
    vq = wl.allocation[0] == "nova-vq"
    extra = {}
    if vq:
        alloc, bk, bv, cwk, cwv = calibrate_vq(wl)
        extra = {"codebook_k": torch.from_numpy(np.concatenate(cwk).view(np.int32)).to(dev),
                 "codebook_v": torch.from_numpy(np.concatenate(cwv).view(np.int32)).to(dev), "query_basis_k": True}
    else:
        alloc, bk, bv = calibrate(wl)
    T = wl.encode_tokens or wl.context
    B, H, d = wl.batch, wl.n_kv_heads, wl.head_dim
    lay = K.Layout(H, wl.n_q_heads, B, T, alloc, **extra)
    pk = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bk])).to(dev)
    pv = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bv])).to(dev)
    nb = min(block, T)
    reps_t = (T + nb - 1) // nb
    kx = torch.from_numpy(W.kv_array(wl, "K", 0, nb)).to(dev).repeat(1, 1, reps_t, 1)[:, :, :T].contiguous()
    vx = torch.from_numpy(W.kv_array(wl, "V", 0, nb)).to(dev).repeat(1, 1, reps_t, 1)[:, :, :T].contiguous()
    ck = torch.empty(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device=dev)
    cv = torch.empty(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device=dev)
    K.kv_encode(lay, kx, vx, T, 0, pk, pv, ck, cv)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        K.kv_encode(lay, kx, vx, T, 0, pk, pv, ck, cv)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    in_bytes = 2 * B * H * T * d * kx.element_size()
    out_bytes = (ck.numel() + cv.numel()) * 4
    del kx, vx, ck, cv
    torch.cuda.empty_cache()
    return {"tokens_per_seq": T, "batch": B, "allocation": [list(a) for a in alloc], "ms": round(ms, 4),
            "input_GB_per_s": round(in_bytes / ms / 1e6, 1),
            "hbm_GB_per_s": round((in_bytes + out_bytes) / ms / 1e6, 1),
            "pct_of_hbm_peak": round(100 * (in_bytes + out_bytes) / ms / 1e6 / HBM_PEAK_GBS, 2)}


def decode_rate(K, wl, block=4096, steps=200, warmup=200, min_bytes=1.0e9, ragged=None, static=False,
                page=0, rope=False):
    """Sustained kv_append_attend_decode throughput of another decode layout at its full size.

    The caches hold the workload's generated keys and values of the first `block` tokens
    repeated along the token axis (same per-token statistics), encoded on the GPU; enough
    layer caches rotate to exceed the Infinity Cache.  Not checked against anything here:
    the GPU parity tests cover these layouts.  ragged: fractions of the context, one per
    sequence, timed as kv_attend_decode_ragged (attention only) over those lengths.
    static: header-free records with each head's fixed quantizer from calibration.
    page: paged caches with pages of this many tokens, the pool holding exactly the
    sequences' pages, assigned by a seeded permutation.  rope: the keys are compressed
    before RoPE (kv_append_attend_decode_rope, LLaMA-3's inverse frequencies, base 500000);
    the line adds the key reconstruction's useful matrix-core rate (2 * 128 * r_K flops
    per token and KV head)."""
    import torch

    from decode_attention_04_amd import calib

    vq = wl.allocation[0] == "nova-vq"
    dev = torch.device("cuda:0")
    if vq:
        alloc, bk, bv, cwk, cwv = calibrate_vq(wl)
    else:
        alloc, bk, bv = calibrate(wl)
    T = wl.context + 1
    B, H, hq, d = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    extra_lay = {}
    if static:
        extra_lay = {"scale_k": [calib.static_scale_word(W.covariance(wl, "K", h), bk[h], alloc[h][1])
                                 for h in range(H)],
                     "scale_v": [calib.static_scale_word(W.covariance(wl, "V", h), bv[h], alloc[h][3])
                                 for h in range(H)]}
    if vq:
        extra_lay = {"codebook_k": torch.from_numpy(np.concatenate(cwk).view(np.int32)).to(dev),
                     "codebook_v": torch.from_numpy(np.concatenate(cwv).view(np.int32)).to(dev)}
    cap = T
    if page:
        cap = (T + page - 1) // page * page
        pps = cap // page
        perm = np.random.default_rng(77).permutation(B * pps).reshape(B, pps).astype(np.int32)
        extra_lay.update(page_tokens=page, pool_pages=B * pps, block_table=torch.from_numpy(perm).to(dev))
    lay = K.Layout(H, hq, B, cap, alloc, **extra_lay, query_basis_k=wl.allocation[0] in ("nova", "nova-vq"))
    pk = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bk])).to(dev)
    pv = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bv])).to(dev)
    reps_t = (T - 1 + block - 1) // block
    kx = torch.from_numpy(W.kv_array(wl, "K", 0, block)).to(dev).repeat(1, 1, reps_t, 1)[:, :, :T - 1].contiguous()
    vx = torch.from_numpy(W.kv_array(wl, "V", 0, block)).to(dev).repeat(1, 1, reps_t, 1)[:, :, :T - 1].contiguous()
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device=dev)
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device=dev)
    K.kv_encode(lay, kx, vx, T - 1, 0, pk, pv, ck, cv)
    k1 = kx[:, :, -1].contiguous()
    v1 = vx[:, :, -1].contiguous()
    del kx, vx
    cache_bytes = (ck.numel() + cv.numel()) * 4
    n_rep = max(2, int(math.ceil(min_bytes / cache_bytes)))
    caches = [(ck, cv)] + [(ck.clone(), cv.clone()) for _ in range(n_rep - 1)]
    q = torch.from_numpy(W.query_array(wl, 0)).to(dev)
    out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    ws_bytes = K.kv_workspace_bytes_rope(lay, T) if rope else K.kv_workspace_bytes(lay, T)
    ws = torch.zeros(ws_bytes // 4, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    inv_freq = torch.from_numpy(500000.0 ** (-np.arange(0, d, 2, dtype=np.float64) / d)).to(dev) if rope else None
    lens = [int(T * f) for f in ragged] if ragged else None
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev) if ragged else None

    def step(i):
        ck_, cv_ = caches[i % n_rep]
        if ragged:
            K.kv_attend_decode_ragged(lay, q, lens_d, T, pk, pv, ck_, cv_, scale, out, ws)
        elif rope:
            K.kv_append_attend_decode_rope(lay, k1, v1, q, T, pk, pv, ck_, cv_, scale, inv_freq, out, ws)
        else:
            K.kv_append_attend_decode(lay, k1, v1, q, T, pk, pv, ck_, cv_, scale, out, ws)

    # at least `warmup` steps and 30 ms of them: after the set-up's idle the first
    # milliseconds of sustained load run slower while the clocks settle
    i, t_w = 0, time.perf_counter()
    while i < warmup or time.perf_counter() - t_w < 0.03:
        step(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    attend_bytes, append_bytes = step_bytes(wl, alloc, T, static)
    if ragged:  # the records of each sequence's own tokens, no append
        rec = attend_bytes - step_bytes(wl, alloc, 0)[0]
        attend_bytes = attend_bytes - rec + rec * sum(lens) // (B * T)
        append_bytes = 0
    gbs = (attend_bytes + append_bytes) / (us * 1e-6) / 1e9
    del caches, ck, cv
    torch.cuda.empty_cache()
    extra = {"lengths": lens, "step": "kv_attend_decode_ragged (no append)"} if ragged else {}
    if static:
        extra["records"] = "header-free (one fixed quantizer per head)"
    if vq:
        extra["records"] = "vector-quantized coordinate pairs (scale word, one index per pair)"
    if rope:
        extra["keys"] = "compressed before RoPE, turned by position at decode (inverse frequencies base 500000)"
        flops = 2.0 * 128 * B * T * sum(a[0] for a in alloc)
        extra["key_reconstruction_TFLOP_per_s"] = round(flops / (us * 1e-6) / 1e12, 1)
    if page:
        extra["paged"] = f"pages of {page} tokens, block table a seeded permutation"
    kclass = K.kv_attend_plan(lay, T)[0]
    kname = "generic" if kclass < 0 else (f"budget class {kclass}" if kclass < 6 else
                                          "vector-quantized class" if kclass == 6 else "frozen layout class")
    return {**extra, "batch": B, "n_q_heads": hq, "n_kv_heads": H, "context_tokens": T,
            "allocation": [list(a) for a in alloc],
            "kernel": "pre-RoPE key kernel" if rope else kname,
            "us_per_step": round(us, 2), "GB_per_s": round(gbs, 1),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "layer_caches_rotated": n_rep}


def measure_distortion(K, wl, heads, n_tokens, formats, static=False):
    """Relative reconstruction distortion sum_t ||x_t - x^_t||^2 / sum_t ||x_t||^2 of KV heads
    `heads` of `wl` (keys and values, the first n_tokens of sequence 0), at each (rank,
    bits) of `formats`, for records the library writes (kv_encode) and reconstructs
    (kv_decode) on the GPU.  Bases: the MSE-ordered eigenvectors of each head's
    covariance with the seeded Hadamard signs folded in; static: header-free records with
    each head's fixed quantizer.  Returns {(head, tensor, (rank, bits)): D}."""
    import torch

    from decode_attention_04_amd import calib

    dev = torch.device("cuda:0")
    n = len(heads)
    x = {t: torch.from_numpy(np.stack([W.tokens(wl, t, 0, h, 0, n_tokens, wl.dtype) for h in heads])[None]).to(dev)
         for t in "KV"}
    energy = {t: (x[t].double() ** 2).sum(dim=(0, 2, 3)) for t in "KV"}
    dirs = {t: [calib.sorted_directions(W.covariance(wl, t, h))[1] for h in heads] for t in "KV"}
    out = {}
    for r, b in formats:
        bases = {t: [calib.fold(dirs[t][i], r, W.hadamard_signs(wl, t, h, r)) for i, h in enumerate(heads)]
                 for t in "KV"}
        scales = {}
        if static:
            scales = {f"scale_{t.lower()}": [calib.static_scale_word(W.covariance(wl, t, h), bases[t][i], b)
                                             for i, h in enumerate(heads)] for t in "KV"}
        lay = K.Layout(n, n, 1, n_tokens, [(r, b, r, b)] * n, **scales)
        pd = {t: torch.from_numpy(calib.concat(bases[t])).to(dev) for t in "KV"}
        ck = torch.empty(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device=dev)
        cv = torch.empty(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device=dev)
        K.kv_encode(lay, x["K"], x["V"], n_tokens, 0, pd["K"], pd["V"], ck, cv)
        for which, t, cache in ((0, "K", ck), (1, "V", cv)):
            rec = torch.empty((1, n, n_tokens, wl.head_dim), dtype=torch.float32, device=dev)
            K.kv_decode(lay, which, n_tokens, 0, pd[t], cache, rec)
            err = ((x[t].double() - rec.double()) ** 2).sum(dim=(0, 2, 3)) / energy[t]
            for i, h in enumerate(heads):
                out[(h, t, (r, b))] = float(err[i])
    return out


def distortion_rate(K, wl=None, tokens=4096):
    """Distortion against bits on 256 synthetic KV heads shaped like the whole LLaMA-3.1-8B
    model's (32 layers x 8), measured on the library's own records: the relative
    reconstruction distortion at full rank for b = 2..8 (quantization alone) with
    per-token headers and header-free, the rate exponent alpha of D ~ 2^(-alpha b)
    fitted per head (least squares of -log2 D over b = 2..8, and from b = 2 to 3), the
    allocation model's D(r, b) = (sum_{i>r} lam_i + q(b) sum_{i<=r} lam_i) / sum lam
    beside it, and the spread max/min of the per-head distortion at the uniform 2
    bits/dim formats (128, 2), (64, 4), (32, 8)."""
    wl = wl or W.LLAMA_256_HEADS
    bits = list(range(2, 9))
    full = [(128, b) for b in bits]
    uni = [(128, 2), (64, 4), (32, 8)]
    D, Ds = {}, {}
    for l0 in range(0, wl.n_kv_heads, 8):
        heads = list(range(l0, min(l0 + 8, wl.n_kv_heads)))
        D.update(measure_distortion(K, wl, heads, tokens, full + uni[1:]))
        Ds.update(measure_distortion(K, wl, heads, tokens, full, static=True))
    H = wl.n_kv_heads

    def exponents(src, t):
        y = np.array([[-np.log2(src[(h, t, (128, b))]) for b in bits] for h in range(H)])
        slope = np.polyfit(np.array(bits, np.float64), y.T, 1)[0]
        local = y[:, 1] - y[:, 0]
        return {"fit_b2_to_b8_mean": round(float(slope.mean()), 3), "fit_min": round(float(slope.min()), 3),
                "fit_max": round(float(slope.max()), 3), "b2_to_b3_mean": round(float(local.mean()), 3)}

    def model(t, r, b):
        lam = np.array([np.sort(np.linalg.eigvalsh(W.covariance(wl, t, h)))[::-1] for h in range(H)])
        return float(np.mean((lam[:, r:].sum(1) + 2.0 ** (-2 * b) / 12 * lam[:, :r].sum(1)) / lam.sum(1)))

    rep = {"workload": wl.name, "heads": H, "tokens_per_head": tokens,
           "bits": bits,
           "full_rank_mean_D": {t: [float(np.mean([D[(h, t, (128, b))] for h in range(H)])) for b in bits]
                                for t in "KV"},
           "full_rank_mean_D_header_free": {t: [float(np.mean([Ds[(h, t, (128, b))] for h in range(H)]))
                                                for b in bits] for t in "KV"},
           "model_full_rank_D": {t: [model(t, 128, b) for b in bits] for t in "KV"},
           "rate_exponent": {t: exponents(D, t) for t in "KV"},
           "rate_exponent_header_free": {t: exponents(Ds, t) for t in "KV"},
           "spread_uniform_2bpd": {}}
    for r, b in uni:
        rep["spread_uniform_2bpd"][f"r{r}b{b}"] = {
            t: {"max_over_min": round(max(D[(h, t, (r, b))] for h in range(H)) /
                                      min(D[(h, t, (r, b))] for h in range(H)), 2),
                "mean_D": float(np.mean([D[(h, t, (r, b))] for h in range(H)])),
                "model_mean_D": model(t, r, b)} for t in "KV"}
    return rep


def logit_error(K, wl=None, tokens=4096, n_queries=256):
    """Relative attention-logit error sum (q . (k - k^))^2 / sum (q . k)^2 of the keys the
    library encodes and reconstructs (kv_encode, kv_decode), for queries drawn from each
    head's generated query distribution: the attention-aware transform (P_K encodes,
    keys reconstructed through Q_K) against the orthonormal basis ordered by attention-KL
    weights, both with the attention-aware allocation's (rank, bits) per head.  The
    comparison the NOVA-KV review proposes as the test of the non-orthogonal transform."""
    import torch

    from decode_attention_04_amd import calib

    wl = wl or W.llama_t128k_nova(2.0)
    dev = torch.device("cuda:0")
    alloc, kblocks, _ = calibrate(wl)
    H = wl.n_kv_heads
    x = torch.from_numpy(np.stack([W.tokens(wl, "K", 0, h, 0, tokens, wl.dtype) for h in range(H)])[None]).to(dev)
    rng = np.random.default_rng(7)
    out = {"workload": wl.name, "tokens_per_head": tokens, "queries_per_head": n_queries}
    for name in ("attention-aware", "orthonormal-kl"):
        if name == "attention-aware":
            keys = [torch.from_numpy(b) for b in kblocks]
            pair = True
        else:
            keys = [torch.from_numpy(calib.fold(calib.sorted_directions(W.covariance(wl, "K", h),
                                                                         W.query_covariance(wl, h))[1], alloc[h][0],
                                                W.hadamard_signs(wl, "K", h, alloc[h][0])).reshape(-1))
                    for h in range(H)]
            pair = False
        lay = K.Layout(H, H, 1, tokens, [(a[0], a[1], a[0], a[1]) for a in alloc], query_basis_k=pair)
        kb = torch.cat(keys).to(dev)
        ck = torch.empty(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device=dev)
        cv = torch.empty(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device=dev)
        vb = torch.zeros(sum(128 * a[0] for a in alloc), dtype=torch.float32, device=dev)
        K.kv_encode(lay, x, x, tokens, 0, kb, vb, ck, cv)
        rec = torch.empty((1, H, tokens, wl.head_dim), dtype=torch.float32, device=dev)
        K.kv_decode(lay, 0, tokens, 0, kb, ck, rec)
        errs = []
        for h in range(H):
            qs = torch.from_numpy(rng.multivariate_normal(np.zeros(wl.head_dim), W.query_covariance(wl, h),
                                                          n_queries)).to(dev)
            kx = x[0, h].double()
            num = ((qs @ (kx - rec[0, h].double()).T) ** 2).sum()
            den = ((qs @ kx.T) ** 2).sum()
            errs.append(float(num / den))
        out[name] = {"per_head": [round(e, 6) for e in errs], "mean": float(np.mean(errs))}
    out["allocation"] = [list(a[:2]) for a in alloc]
    return out


def _cpu_workers() -> int:
    """Host cores the oracle runs on: every core this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_worker(kind, wl, alloc, bk, bv, T, units, barrier, results):
    """One oracle worker process (one BLAS thread): prepare its units untimed, wait for
    the others, then time its share.  kind "attend": encode each (sequence, KV head)
    unit's records, then time the attention of its query heads over them; kind
    "encode": generate each unit's keys and values, then time their encode."""
    from threadpoolctl import threadpool_limits

    from oracle import attention, codec

    with threadpool_limits(limits=1):
        prepared = []
        for b, h in units:
            rk, b_k, rv, b_v = alloc[h]
            xk = W.tokens(wl, "K", b, h, 0, T)
            xv = W.tokens(wl, "V", b, h, 0, T)
            if kind == "attend":
                rec_k = np.concatenate([codec.encode_tokens(xk[i:i + 16384], bk[h], b_k) for i in range(0, T, 16384)])
                rec_v = np.concatenate([codec.encode_tokens(xv[i:i + 16384], bv[h], b_v) for i in range(0, T, 16384)])
                prepared.append((b, h, rec_k, rec_v))
            else:
                prepared.append((b, h, W.cast(xk, wl.dtype), W.cast(xv, wl.dtype)))
        q = W.query_array(wl, 0).astype(np.float64) if kind == "attend" else None
        scale = 1.0 / math.sqrt(wl.head_dim)
        g = wl.group
        barrier.wait()
        t0 = time.perf_counter()
        nbytes = 0
        for b, h, u, v in prepared:
            rk, b_k, rv, b_v = alloc[h]
            if kind == "attend":
                attention.attend_head_records(q[b, h * g:(h + 1) * g], bk[h], u, rk, b_k, bv[h], v, rv, b_v, scale)
                nbytes += u.nbytes + v.nbytes
            else:
                rec_k = codec.encode_tokens(u, bk[h], b_k)
                rec_v = codec.encode_tokens(v, bv[h], b_v)
                nbytes += u.nbytes + v.nbytes + rec_k.nbytes + rec_v.nbytes
        t1 = time.perf_counter()
    results.put((t0, t1, nbytes, len(prepared)))


def _oracle_pool(kind, wl, alloc, bk, bv, T, units):
    """Run the oracle over `units` on every host core at once (fork workers, started
    before this process touches the GPU); wall time from the first start to the last end."""
    import multiprocessing as mp

    ctx = mp.get_context("fork")
    n = min(_cpu_workers(), len(units))
    barrier = ctx.Barrier(n)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(kind, wl, alloc, bk, bv, T, units[i::n], barrier, results))
             for i in range(n)]
    for p in procs:
        p.start()
    res = [results.get() for _ in procs]
    for p in procs:
        p.join()
        if p.exitcode != 0:
            raise RuntimeError(f"oracle worker exited with {p.exitcode}")
    wall = max(r[1] for r in res) - min(r[0] for r in res)
    return wall, sum(r[2] for r in res), sum(r[3] for r in res), n


def cpu_baseline(wl, alloc, bk, bv, T):
    """The oracle (float64 numpy) on the host's cores: one worker process per core
    (at most 16), one BLAS thread each, work split by (sequence, KV head) unit.
    Timed: the decode attention of every unit of the workload (its query heads over
    its T records; records encoded beforehand, untimed), and the encode of the
    Qwen-shaped layer's 4096-token prefill chunk (8 sequences x 4 KV heads, keys and
    values)."""
    units = [(b, h) for b in range(wl.batch) for h in range(wl.n_kv_heads)]
    wall, nbytes, done, n = _oracle_pool("attend", wl, alloc, bk, bv, T, units)
    ewl = W.QWEN_T128K
    ealloc, ebk, ebv = calibrate(ewl)
    eunits = [(b, h) for b in range(ewl.batch) for h in range(ewl.n_kv_heads)]
    ewall, ebytes, _, en = _oracle_pool("encode", ewl, ealloc, ebk, ebv, ewl.encode_tokens, eunits)
    return {
        "value": round(nbytes / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "sample": f"all {done} (sequence, KV head) units of the workload, attention of each unit's {wl.group} "
                  f"query heads over its {T} records ({nbytes / 1e6:.1f} MB of records) on {n} worker processes "
                  f"(one BLAS thread each): {wall:.2f} s wall; records encoded beforehand, untimed",
        "seconds": round(wall, 3),
        "encode": {"workload": ewl.name, "tokens_per_seq": ewl.encode_tokens, "units": len(eunits),
                   "cores": en, "seconds": round(ewall, 3),
                   "GB_per_s": round(ebytes / ewall / 1e9, 4),
                   "bytes": int(ebytes), "note": "fp16 keys and values read plus records written, per second"},
    }


def phase_stamps(K, wl, reps=20, warmup=200, block=4096):
    """Per-phase times of the fused decode step's workgroups, from the diagnostic build's
    stamps (100 MHz real-time counter, 10 ns): the same launch configuration as the
    benchmark on caches holding the workload's first `block` tokens repeated (same
    per-token statistics), rotated over layer copies as in decode_rate.  Returns a
    markdown summary: the launch timeline (when the last workgroup passes each phase)
    and the per-workgroup phase durations (median, 90th percentile, maximum over the
    workgroups, medians over `reps` launches)."""
    import ctypes

    import torch

    lib = K.raw()
    if not hasattr(lib, "kv_debug_stamps"):
        raise SystemExit("the loaded library has no phase stamps: build it with "
                         "`python -m decode_attention_04_amd.build --stamps` and set KVTC_LIBRARY")
    alloc, bk, bv = calibrate(wl)
    T = wl.context + 1
    B, H, hq, d = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    lay = K.Layout(H, hq, B, T, alloc)
    kclass, ns, grid = K.kv_attend_plan(lay, T)
    dev = torch.device("cuda:0")
    pk = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bk])).to(dev)
    pv = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bv])).to(dev)
    reps_t = (T - 1 + block - 1) // block
    kx = torch.from_numpy(W.kv_array(wl, "K", 0, block)).to(dev).repeat(1, 1, reps_t, 1)[:, :, :T - 1].contiguous()
    vx = torch.from_numpy(W.kv_array(wl, "V", 0, block)).to(dev).repeat(1, 1, reps_t, 1)[:, :, :T - 1].contiguous()
    ck = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device=dev)
    cv = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device=dev)
    K.kv_encode(lay, kx, vx, T - 1, 0, pk, pv, ck, cv)
    k1, v1 = kx[:, :, -1].contiguous(), vx[:, :, -1].contiguous()
    del kx, vx
    n_rep = max(2, int(math.ceil(1.0e9 / ((ck.numel() + cv.numel()) * 4))))
    caches = [(ck, cv)] + [(ck.clone(), cv.clone()) for _ in range(n_rep - 1)]
    q = torch.from_numpy(W.query_array(wl, 0)).to(dev)
    out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device=dev)
    st = torch.zeros((grid, 32), dtype=torch.int64, device=dev)
    lib.kv_debug_stamps.restype = ctypes.c_int32
    lib.kv_debug_stamps.argtypes = [ctypes.c_void_p]
    scale = 1.0 / math.sqrt(d)
    for i in range(warmup):
        K.kv_append_attend_decode(lay, k1, v1, q, T, pk, pv, *caches[i % n_rep], scale, out, ws)
    runs = []
    lib.kv_debug_stamps(st.data_ptr())
    for i in range(reps):
        st.zero_()
        K.kv_append_attend_decode(lay, k1, v1, q, T, pk, pv, *caches[i % n_rep], scale, out, ws)
        torch.cuda.synchronize()
        runs.append(st.cpu().numpy().astype(np.int64))
    lib.kv_debug_stamps(None)
    us = 0.01  # counter ticks (100 MHz) in microseconds
    tl_names = ["first workgroup starts", "last workgroup starts", "last query projection done",
                "median tile loop done (wave mean)", "last tile loop done", "last split partial stored",
                "last arrival counted", "last split merge done"]
    tl, ph = [], {}
    for s_ in runs:
        t0 = s_[:, 0].min()
        rel = (s_ - t0) * us
        loop_end = rel[:, 2:6]
        tl.append([0.0, rel[:, 0].max(), rel[:, 1].max(), np.median(loop_end.mean(1)), loop_end.max(),
                   rel[:, 6].max(), rel[:, 7].max(), rel[s_[:, 8] > 0, 8].max()])
        app0 = s_[:, 11] > 0  # appending workgroups: their projection starts after the encode
        durs = {
            "start after the first workgroup": rel[:, 0],
            "query projection (and first tile copies issued)": rel[:, 1] - rel[:, 0],
            "  to the start of the projection (head, split and buffer set-up)": (rel[:, 28] - rel[:, 0])[~app0],
            "    head and its descriptor": (rel[:, 29] - rel[:, 0])[~app0],
            "    split bounds": (rel[:, 30] - rel[:, 29])[~app0],
            "    buffers and tile areas": (rel[:, 31] - rel[:, 30])[~app0],
            "    format dispatch to the projection start": (rel[:, 28] - rel[:, 31])[~app0],
            "  basis and query loads, first tile copies issued": (rel[:, 24] - rel[:, 28])[~app0],
            "  queries staged (their loads complete)": (rel[:, 25] - rel[:, 24])[s_[:, 24] > 0],
            "  projection (basis loads complete)": (rel[:, 26] - rel[:, 25])[s_[:, 24] > 0],
            "  exponents and sums": (rel[:, 27] - rel[:, 26])[s_[:, 24] > 0],
            "  operands built": (rel[:, 1] - rel[:, 27])[s_[:, 24] > 0],
            "tile loop, per wave": (loop_end - rel[:, 1:2]).reshape(-1),
            "wave spread (last wave - first wave of a workgroup)": loop_end.max(1) - loop_end.min(1),
            "wave merge, back-projection, partial stores (from the last wave)": rel[:, 6] - loop_end.max(1),
            "  wave partials staged in LDS (from the last wave)": rel[:, 12] - loop_end.max(1),
            "    per wave: tile loop end to partial in LDS": (rel[:, 16:20] - loop_end).reshape(-1),
            "    per wave: P_V row loads issued": (rel[:, 20:24] - rel[:, 16:20]).reshape(-1),
            "    last wave's loads issued to the barrier passed": rel[:, 12] - rel[:, 20:24].max(1),
            "  wave merge": rel[:, 13] - rel[:, 12],
            "  back-projection, partial stores issued": rel[:, 14] - rel[:, 13],
            "  partial stores completed": rel[:, 6] - rel[:, 14],
            "arrival atomic": rel[:, 7] - rel[:, 6],
            "split merge (merging workgroups)": (rel[:, 8] - rel[:, 7])[s_[:, 8] > 0],
        }
        for k, v in durs.items():
            ph.setdefault(k, []).append((np.median(v), np.percentile(v, 90), v.max()))
        app = s_[:, 11] > 0  # the workgroups that encode the appended token first
        hw = s_[:, 9]
        cu = (s_[:, 10] << 8) | ((hw >> 8) & 0xFF)  # XCC, then shader engine / array / CU bits of HW_ID
        order = np.zeros(len(s_), np.int64)
        for key in np.unique(cu):
            idx = np.flatnonzero(cu == key)
            order[idx[np.argsort(s_[idx, 0], kind="stable")]] = np.arange(len(idx))
        extra = {
            "appending workgroups: append encode": rel[app, 11] - rel[app, 0],
            "appending workgroups: query projection after the append": rel[app, 1] - rel[app, 11],
            "appending workgroups: tile loop end": loop_end[app].max(1),
            "other workgroups: tile loop end": loop_end[~app].max(1),
        }
        for rank in range(int(order.max()) + 1):
            extra[f"workgroups dispatched {rank + 1}. on their CU: tile loop, per wave"] = \
                (loop_end[order == rank] - rel[order == rank, 1:2]).reshape(-1)
        for k, v in extra.items():
            if len(v):
                ph.setdefault(k, []).append((np.median(v), np.percentile(v, 90), v.max()))
    tl = np.median(np.array(tl), axis=0)
    lines = [f"Workload {wl.name}: kernel class {kclass}, {grid} workgroups, {ns} splits per "
             f"(sequence, KV head); {reps} stamped launches after {warmup} unstamped ones, medians.", "",
             "| launch timeline (last workgroup to pass) | us after the first workgroup starts |", "|---|---:|"]
    lines += [f"| {n} | {v:.2f} |" for n, v in zip(tl_names, tl)]
    lines += ["", "| phase, per workgroup | median (us) | p90 (us) | max (us) |", "|---|---:|---:|---:|"]
    for k, v in ph.items():
        m = np.median(np.array(v), axis=0)
        lines.append(f"| {k} | {m[0]:.2f} | {m[1]:.2f} | {m[2]:.2f} |")
    return "\n".join(lines)


def sources_digest() -> str:
    """sha256 over the HIP/C++ sources of the library (which code a counter profile belongs to)."""
    import hashlib

    csrc = os.path.join(ROOT, "decode_attention_04_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".h", ".hip", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def profile_fields(name: str):
    """The machine-readable fields ("- key: `value`" lines) of a committed profile summary,
    or None when it is missing or was taken on other library sources."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("sources_sha256") != sources_digest():
        return None
    return fields


def measured_traffic(workload: str):
    """HBM bytes per append + attend launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size)
    from the committed counter profile of this workload, if it was taken on these sources."""
    f = profile_fields(f"traffic_append_attend_{workload}.md")
    return int(f["traffic_bytes_per_launch"]) if f else None


def measured_busy(workload: str):
    """Share of the SIMD cycles of a decode launch spent issuing VALU, matrix-core and LDS
    instructions, from the committed SQ counter profile of this workload (same source check)."""
    f = profile_fields(f"sq_append_attend_{workload}.md")
    if not f:
        return None
    return {k: float(f[k]) for k in ("valu_issue_pct", "mfma_busy_pct", "lds_issue_pct")} | \
        {"source": f"profiles/sq_append_attend_{workload}.md"}


def read_ceiling(nbytes: int, reps: int = 100):
    """The GPU's own streaming-read rate: libkvtc_probe.so's plain read of nbytes (the
    decode step's bytes), four buffers rotated (beyond the Infinity Cache), back to back,
    at a few grid sizes; the best rate in GB/s and its grid.  A reference for the decode
    kernels beside the datasheet peak."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "decode_attention_04_amd", "libkvtc_probe.so"))
    fn = lib.kvtc_read_probe
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    n = (nbytes // 16) * 16
    bufs = [torch.ones(n // 4, dtype=torch.int32, device="cuda") for _ in range(4)]
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = (0.0, 0)
    for wgs in (768, 2048, 8192):
        def launch(i):
            rc = fn(bufs[i % 4].data_ptr(), n, wgs, sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"read probe launch failed ({rc})")
        i, t_w = 0, time.perf_counter()  # 30 ms of load first, as for the decode rates
        while i < 20 or time.perf_counter() - t_w < 0.03:
            launch(i)
            i += 1
            if i % 50 == 0:
                torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            launch(i)
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = n / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
        best = max(best, (gbs, wgs))
    del bufs
    torch.cuda.empty_cache()
    return {"GB_per_s": round(best[0], 1), "pct_of_hbm_peak": round(100 * best[0] / HBM_PEAK_GBS, 2),
            "workgroups": best[1], "bytes": n,
            "probe": "plain 16-byte non-temporal reads, four buffers rotated, back-to-back launches"}


def copy_probe(mib: int):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counter readings."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: 3 copies of {mib} MiB ({n * 4} bytes read and written each)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the timed steps start from the steady state of back-to-back launches (clocks
    # and caches settled); isolated launches vary more (single_launch_us reports
    # their p10 / p50 / p90); 200 steps take about 16 ms
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama-128k-2bpd")
    ap.add_argument("--replica-bytes", type=float, default=1.2e9, help="total bytes of rotated layer caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-rates", action="store_true",
                    help="skip the decode measurements of the other layouts (128K budgets, Qwen, 32K batch 16)")
    ap.add_argument("--no-encode-rates", action="store_true",
                    help="skip the prefill encode measurements of the prefill workloads")
    ap.add_argument("--no-distortion", action="store_true",
                    help="skip the distortion-rate characterisation of the 256 synthetic KV heads")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a captured HIP graph per step instead of eager launches")
    ap.add_argument("--phase-stamps", type=int, default=0, metavar="REPS",
                    help="only run REPS launches of the decode step with the phase-stamp build "
                         "(libkvtc_stamps.so) and print the per-phase timing summary")
    ap.add_argument("--decode-layout", default="", metavar="NAME",
                    help="only time one other decode layout (pre-rope-2bpd, pre-rope-0.5bpd, vq-2bpd, paged-2bpd, b1-t32k, "
                         "0.5bpd, 4bpd) "
                         "with --steps / --warmup launches and print its line (for counter profiles)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 3 times (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.decode_layout:
        import decode_attention_04_amd as K
        layouts = {
            "pre-rope-2bpd": lambda: decode_rate(K, W.llama_t128k(2.0), steps=args.steps, warmup=args.warmup, rope=True),
            "pre-rope-0.5bpd": lambda: decode_rate(K, W.llama_t128k(0.5), steps=args.steps, warmup=args.warmup,
                                                   rope=True),
            "vq-2bpd": lambda: decode_rate(K, W.llama_t128k_nova_vq(2.0), steps=args.steps, warmup=args.warmup),
            "paged-2bpd": lambda: decode_rate(K, W.llama_t128k(2.0), steps=args.steps, warmup=args.warmup, page=256),
            "b1-t32k": lambda: decode_rate(K, W.LLAMA_T32K, steps=args.steps, warmup=args.warmup),
            "0.5bpd": lambda: decode_rate(K, W.llama_t128k(0.5), steps=args.steps, warmup=args.warmup),
            "4bpd": lambda: decode_rate(K, W.llama_t128k(4.0), steps=args.steps, warmup=args.warmup),
        }
        if args.decode_layout not in layouts:
            raise SystemExit(f"unknown decode layout {args.decode_layout}; choose from {sorted(layouts)}")
        print(json.dumps(layouts[args.decode_layout]()), flush=True)
        return
    if args.phase_stamps:
        os.environ["KVTC_LIBRARY"] = os.path.join(ROOT, "decode_attention_04_amd", "libkvtc_stamps.so")
        import decode_attention_04_amd._lib as K
        print(phase_stamps(K, pick_workload(args.workload), reps=args.phase_stamps))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the decode step is measured on one GPU; --gpus must be 1 (a sharded layout splits the KV heads across GPUs, each running this same kernel on its share)"}))
        raise SystemExit(2)

    wl = pick_workload(args.workload)
    T = wl.context
    B, hkv, hq, d = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    t_setup = time.time()
    alloc, bk, bv = calibrate(wl)
    log(f"workload {wl.name}: allocation (rk, bk, rv, bv) per KV head {alloc}")
    # the oracle's CPU baseline first: its worker processes fork before this process touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, alloc, bk, bv, T + 1)
        log(f"cpu baseline (oracle): {cpu}")

    import torch

    import decode_attention_04_amd as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lay = K.Layout(hkv, hq, B, T + 1, alloc)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if wl.dtype == "f32" else torch.float16
    pk = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bk])).to(dev)
    pv = torch.from_numpy(np.concatenate([p.reshape(-1) for p in bv])).to(dev)

    # prefill: keys/values of the context, encoded on the GPU
    ck0 = torch.zeros(K.kv_cache_bytes(lay, 0) // 4, dtype=torch.int32, device=dev)
    cv0 = torch.zeros(K.kv_cache_bytes(lay, 1) // 4, dtype=torch.int32, device=dev)
    chunk = max(1, (1 << 15))
    enc_ms = 0.0
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        kx = torch.from_numpy(W.kv_array(wl, "K", t0, n)).to(dev)
        vx = torch.from_numpy(W.kv_array(wl, "V", t0, n)).to(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        K.kv_encode(lay, kx, vx, n, t0, pk, pv, ck0, cv0)
        e1.record()
        torch.cuda.synchronize()
        enc_ms += e0.elapsed_time(e1)
        del kx, vx
    enc_in_bytes = 2 * B * hkv * T * d * (4 if wl.dtype == "f32" else 2)
    cache_bytes = (ck0.numel() + cv0.numel()) * 4
    n_rep = max(2, int(math.ceil(args.replica_bytes / cache_bytes)))
    caches = [(ck0, cv0)] + [(ck0.clone(), cv0.clone()) for _ in range(n_rep - 1)]
    k_new = torch.from_numpy(W.kv_array(wl, "K", T, 1)[:, :, 0]).to(dev)
    v_new = torch.from_numpy(W.kv_array(wl, "V", T, 1)[:, :, 0]).to(dev)
    q = torch.from_numpy(W.query_array(wl, 0)).to(dev)
    out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kv_workspace_bytes(lay, T + 1) // 4, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f} s; {n_rep} layer caches of {cache_bytes / 1e6:.1f} MB; "
        f"GPU encode of the {T}-token prefill: {enc_ms:.3f} ms ({enc_in_bytes / enc_ms / 1e6:.1f} GB/s of fp input)")

    stream = torch.cuda.current_stream()

    def step(i):
        ck, cv = caches[i % n_rep]
        K.kv_append_attend_decode(lay, k_new, v_new, q, T + 1, pk, pv, ck, cv, scale, out, ws)

    # the step as two calls on every cache first: the fused launch must reproduce it bit for bit
    for ck, cv in caches:
        K.kv_append(lay, k_new, v_new, T, pk, pv, ck, cv)
        K.kv_attend_decode(lay, q, T + 1, pk, pv, ck, cv, scale, out, ws)
    torch.cuda.synchronize()
    two_call_out = out.clone()
    out.zero_()
    for i in range(n_rep):
        step(i)
    torch.cuda.synchronize()
    ref_out = out.clone()
    assert torch.equal(ref_out, two_call_out), "fused append + attend differs from kv_append + kv_attend_decode"

    # with --graph each timed step replays a HIP graph of that step (one graph per layer
    # cache); by default the step's single launch is issued eagerly, back to back
    graphs = []
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        for i in range(n_rep):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for r in range(2):  # replays agree with the eager step, with eager work in between
            for g in graphs:
                out.zero_()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(out, ref_out), "graph replay differs from the eager step"
            step(r)
            torch.cuda.synchronize()
    def timed_step(i):
        if graphs:
            graphs[i % n_rep].replay()
        else:
            step(i)

    # the warm-up steps run right before the timed ones: the checks above leave the GPU
    # idle for ~0.1 s (first use of torch's comparison kernels), and after such an idle
    # the first milliseconds of sustained load run up to 20% slower while the clocks settle
    for i in range(args.warmup):
        timed_step(i)
    steps = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        timed_step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "timed steps changed the output"
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / steps

    # the same kernel in a longer back-to-back run of its own (after 30 ms of launches,
    # as for the other layouts' rates), reported beside the timed steps
    i, t_w = 0, time.perf_counter()
    while time.perf_counter() - t_w < 0.03:
        ck, cv = caches[i % n_rep]
        K.kv_append_attend_decode(lay, k_new, v_new, q, T + 1, pk, pv, ck, cv, scale, out, ws)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    att_ms = []
    for r in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n_rep * 4):
            ck, cv = caches[i % n_rep]
            K.kv_append_attend_decode(lay, k_new, v_new, q, T + 1, pk, pv, ck, cv, scale, out, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        att_ms.append(e0.elapsed_time(e1) / (n_rep * 4))
    att_avg = float(np.median(att_ms))
    # distribution of single launches: events around each of 100 launches (the events'
    # own gaps are outside each interval)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(100)]
    for i, (e0, e1) in enumerate(ev):
        ck, cv = caches[i % n_rep]
        e0.record(stream)
        K.kv_append_attend_decode(lay, k_new, v_new, q, T + 1, pk, pv, ck, cv, scale, out, ws)
        e1.record(stream)
    torch.cuda.synchronize()
    one = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    pct = {f"p{p}": round(float(np.percentile(one, p)), 2) for p in (10, 50, 90)}
    attend_bytes, append_bytes = step_bytes(wl, alloc, T + 1)
    gbs = (attend_bytes + append_bytes) / (ms_step * 1e-3) / 1e9
    att_gbs = (attend_bytes + append_bytes) / (att_avg * 1e-3) / 1e9
    # the roofline's kernel rate: a step is one launch of the kernel and the timed steps
    # run back to back, so the events around the timed region on the launch stream
    # give the kernel's average launch duration over exactly those launches
    roof_gbs = gbs
    log(f"step {ms_step * 1e3:.1f} us over {steps} steps{' (graph replays)' if graphs else ''}; "
        f"append+attend kernel {att_avg * 1e3:.1f} us (min {min(att_ms) * 1e3:.1f} max {max(att_ms) * 1e3:.1f}); "
        f"{gbs:.1f} GB/s step, {att_gbs:.1f} GB/s kernel ({100 * att_gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})")
    traffic = measured_traffic(wl.name)
    if traffic is not None:
        log(f"HBM traffic per launch from the committed counter profile: {traffic / 1e6:.1f} MB "
            f"(algorithmic {(attend_bytes + append_bytes) / 1e6:.1f} MB)")

    enc_rates = None
    if not args.no_encode_rates:
        enc_rates = {}
        for ewl in (W.llama_prefill(32, 8), W.llama_prefill(64, 4), W.QWEN_T128K,
                    dataclasses.replace(W.llama_t128k_nova_vq(2.0), encode_tokens=4096)):
            enc_rates[ewl.name] = encode_rate(K, ewl)
            log(f"encode {ewl.name}: {enc_rates[ewl.name]}")

    dec_rates = None
    if not args.no_decode_rates:
        dec_rates = {}
        for dwl in (W.llama_t128k(0.5), W.llama_t128k(1.0), W.llama_t128k(4.0), W.QWEN_T128K,
                    W.llama_prefill(32, 8), W.llama_prefill(64, 4), W.llama_t128k_c2(2.0),
                    W.llama_t128k_c2(2.0, "joint"), W.llama_t128k_c2(1.0), W.llama_t128k_nova(2.0), W.LLAMA_T32K,
                    W.llama_t128k_nova_vq(2.0), W.llama_t128k_nova_vq(1.0)):
            dec_rates[dwl.name] = decode_rate(K, dwl)
            log(f"decode {dwl.name}: {dec_rates[dwl.name]}")
        name = W.llama_t128k(2.0).name + "-paged"
        dec_rates[name] = decode_rate(K, W.llama_t128k(2.0), page=256)
        log(f"decode {name}: {dec_rates[name]}")
        for bpd in (0.5, 1.0):
            name = W.llama_t128k(bpd).name + "-header-free"
            dec_rates[name] = decode_rate(K, W.llama_t128k(bpd), static=True)
            log(f"decode {name}: {dec_rates[name]}")
        name = W.llama_t128k(2.0).name + "-ragged"
        dec_rates[name] = decode_rate(K, W.llama_t128k(2.0), ragged=(1.0, 0.75, 0.5, 0.25))
        log(f"decode {name}: {dec_rates[name]}")
        for bpd in (2.0, 0.5):
            name = W.llama_t128k(bpd).name + "-pre-rope-keys"
            dec_rates[name] = decode_rate(K, W.llama_t128k(bpd), rope=True)
            log(f"decode {name}: {dec_rates[name]}")

    ceiling = read_ceiling(attend_bytes + append_bytes)
    log(f"streaming-read ceiling of this GPU: {ceiling}")

    dist = None
    if not args.no_distortion:
        dist = distortion_rate(K)
        dist["attention_logit_error"] = logit_error(K)
        log(f"distortion-rate: {json.dumps(dist)}")

    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": B, "n_q_heads": hq, "n_kv_heads": hkv, "head_dim": d, "context_tokens": T + 1,
            "allocation": [list(a) for a in alloc],
            "step": "kv_append_attend_decode (append of 1 token fused with the attention)",
            "timing": "HIP graph replay per step" if graphs else "one eager launch per step, back to back",
            "layer_caches_rotated": n_rep,
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "hbm_read_ceiling": ceiling,
            "pct_of_read_ceiling": round(100 * gbs / ceiling["GB_per_s"], 2),
            "single_launch_us": pct,
            "context_tokens_per_s": round(B * (T + 1) / (ms_step * 1e-3), 1),
            "bytes_per_step": attend_bytes + append_bytes,
            "encode_prefill_ms": round(enc_ms, 4),
            "encode_rates": enc_rates,
            "other_decode_layouts": dec_rates,
            "distortion_rate": dist,
            "unit_busy_pct": measured_busy(wl.name),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kv_append_attend_decode",
            "achieved": round(roof_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
            "launch_us": round(ms_step * 1e3, 2),
            "back_to_back_run_us": round(att_avg * 1e3, 2),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
