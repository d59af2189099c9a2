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
    from decode_attention_04_amd import calib

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


def step_bytes(wl, alloc, T):
    """Algorithmic HBM bytes of one decode step: attention part and append part."""
    from decode_attention_04_amd import kv_record_words

    B, hq, d = wl.batch, wl.n_q_heads, wl.head_dim
    esz = 4 if wl.dtype == "f32" else 2
    rec = sum(4 * (kv_record_words(a[0], a[1]) + kv_record_words(a[2], a[3])) for a in alloc)
    basis = sum(4 * d * (a[0] + a[2]) for a in alloc)
    attend = B * T * rec + B * hq * d * esz + basis + B * hq * d * 4
    append = B * wl.n_kv_heads * 2 * d * esz + B * rec + basis
    return attend, append


def encode_rate(K, wl, block=2048, reps=5):
    """kv_encode of the workload's prefill chunk (every sequence and KV head at once).

    Inputs: the workload's generated keys and values for the first `block` tokens,
    repeated along the token axis to the chunk length on the GPU (same per-token
    statistics, so the same share of coordinates near a rounding boundary)."""
    import torch

    alloc, bk, bv = calibrate(wl)
    T = wl.encode_tokens or wl.context
    B, H, d = wl.batch, wl.n_kv_heads, wl.head_dim
    lay = K.Layout(H, wl.n_q_heads, B, T, alloc)
    dev = torch.device("cuda:0")
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


def decode_rate(K, wl, block=4096, steps=200, warmup=200, min_bytes=1.0e9, ragged=None):
    """Sustained kv_append_attend_decode throughput of another decode layout at its full size.

    The caches hold the workload's generated keys and values of the first `block` tokens
    repeated along the token axis (same per-token statistics), encoded on the GPU; enough
    layer caches rotate to exceed the Infinity Cache.  Not checked against anything here:
    the GPU parity tests cover these layouts.  ragged: fractions of the context, one per
    sequence, timed as kv_attend_decode_ragged (attention only) over those lengths."""
    import torch

    alloc, bk, bv = calibrate(wl)
    T = wl.context + 1
    B, H, hq, d = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    lay = K.Layout(H, hq, B, T, alloc)
    dev = torch.device("cuda:0")
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
    ws = torch.zeros(K.kv_workspace_bytes(lay, T) // 4, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    lens = [int(T * f) for f in ragged] if ragged else None
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev) if ragged else None

    def step(i):
        ck_, cv_ = caches[i % n_rep]
        if ragged:
            K.kv_attend_decode_ragged(lay, q, lens_d, T, pk, pv, ck_, cv_, scale, out, ws)
        else:
            K.kv_append_attend_decode(lay, k1, v1, q, T, pk, pv, ck_, cv_, scale, out, ws)

    for i in range(warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    attend_bytes, append_bytes = step_bytes(wl, alloc, T)
    if ragged:  # the records of each sequence's own tokens, no append
        rec = attend_bytes - step_bytes(wl, alloc, 0)[0]
        attend_bytes = attend_bytes - rec + rec * sum(lens) // (B * T)
        append_bytes = 0
    gbs = (attend_bytes + append_bytes) / (us * 1e-6) / 1e9
    del caches, ck, cv
    torch.cuda.empty_cache()
    extra = {"lengths": lens, "step": "kv_attend_decode_ragged (no append)"} if ragged else {}
    return {**extra, "batch": B, "n_q_heads": hq, "n_kv_heads": H, "context_tokens": T,
            "allocation": [list(a) for a in alloc], "us_per_step": round(us, 2), "GB_per_s": round(gbs, 1),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "layer_caches_rotated": n_rep}


def cpu_baseline(wl, alloc, bk, bv, T, budget_s=12.0):
    """The oracle (float64 numpy, one BLAS thread) on whole (sequence, KV head) units of the same workload."""
    from threadpoolctl import threadpool_limits

    from oracle import attention, codec

    q = W.query_array(wl, 0).astype(np.float64)
    scale = 1.0 / math.sqrt(wl.head_dim)
    done, secs, nbytes = 0, 0.0, 0
    units = [(b, h) for b in range(wl.batch) for h in range(wl.n_kv_heads)]
    with threadpool_limits(limits=1):
        for b, h in units:
            rk, b_k, rv, b_v = alloc[h]
            xk = W.tokens(wl, "K", b, h, 0, T)
            xv = W.tokens(wl, "V", b, h, 0, T)
            rec_k = np.concatenate([codec.encode_tokens(xk[i:i + 16384], bk[h], b_k) for i in range(0, T, 16384)])
            rec_v = np.concatenate([codec.encode_tokens(xv[i:i + 16384], bv[h], b_v) for i in range(0, T, 16384)])
            g = wl.group
            t0 = time.perf_counter()
            attention.attend_head_records(q[b, h * g:(h + 1) * g], bk[h], rec_k, rk, b_k, bv[h], rec_v, rv, b_v, scale)
            secs += time.perf_counter() - t0
            nbytes += (rec_k.nbytes + rec_v.nbytes)
            done += 1
            if secs >= budget_s:
                break
    return {
        "value": round(nbytes / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {len(units)} (sequence, KV head) units, attention of its {wl.group} query heads "
                  f"over {T} records each ({nbytes / 1e6:.1f} MB of records, {secs:.2f} s); oracle encode not timed",
        "seconds": round(secs, 3),
    }


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


def measured_traffic(workload: str):
    """HBM bytes per append + attend launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size)
    from the committed counter profile of this workload, if it was taken on these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_append_attend_{workload}.md")
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
    return int(fields["traffic_bytes_per_launch"])


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
    # a few hundred back-to-back launches bring the GPU to its sustained clocks (the
    # first ~100 decode launches run up to 10% slower); 200 steps take about 16 ms
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama-128k-2bpd")
    ap.add_argument("--replica-bytes", type=float, default=1.2e9, help="total bytes of rotated layer caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-rates", action="store_true",
                    help="skip the decode measurements of the other layouts (128K budgets, Qwen, 32K batch 16)")
    ap.add_argument("--no-encode-rates", action="store_true",
                    help="skip the prefill encode measurements of the prefill workloads")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a captured HIP graph per step instead of eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 3 times (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the decode step is measured on one GPU; --gpus must be 1 (a sharded layout splits the KV heads across GPUs, each running this same kernel on its share)"}))
        raise SystemExit(2)

    import torch

    import decode_attention_04_amd as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = pick_workload(args.workload)
    T = wl.context
    B, hkv, hq, d = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    t_setup = time.time()
    alloc, bk, bv = calibrate(wl)
    log(f"workload {wl.name}: allocation (rk, bk, rv, bv) per KV head {alloc}")
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
    for i in range(max(args.warmup, n_rep)):
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
    steps = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        if graphs:
            graphs[i % n_rep].replay()
        else:
            step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "timed steps changed the output"
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / steps

    # the step's kernel alone: back-to-back launches on the same stream
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
    attend_bytes, append_bytes = step_bytes(wl, alloc, T + 1)
    gbs = (attend_bytes + append_bytes) / (ms_step * 1e-3) / 1e9
    att_gbs = (attend_bytes + append_bytes) / (att_avg * 1e-3) / 1e9
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
        for ewl in (W.llama_prefill(32, 8), W.llama_prefill(64, 4), W.QWEN_T128K):
            enc_rates[ewl.name] = encode_rate(K, ewl)
            log(f"encode {ewl.name}: {enc_rates[ewl.name]}")

    dec_rates = None
    if not args.no_decode_rates:
        dec_rates = {}
        for dwl in (W.llama_t128k(0.5), W.llama_t128k(1.0), W.llama_t128k(4.0), W.QWEN_T128K,
                    W.llama_prefill(32, 8), W.llama_prefill(64, 4), W.llama_t128k_c2(2.0)):
            dec_rates[dwl.name] = decode_rate(K, dwl)
            log(f"decode {dwl.name}: {dec_rates[dwl.name]}")
        name = W.llama_t128k(2.0).name + "-ragged"
        dec_rates[name] = decode_rate(K, W.llama_t128k(2.0), ragged=(1.0, 0.75, 0.5, 0.25))
        log(f"decode {name}: {dec_rates[name]}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, alloc, bk, bv, T + 1, args.cpu_seconds)
        log(f"cpu baseline (oracle): {cpu}")

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
            "context_tokens_per_s": round(B * (T + 1) / (ms_step * 1e-3), 1),
            "bytes_per_step": attend_bytes + append_bytes,
            "encode_prefill_ms": round(enc_ms, 4),
            "encode_rates": enc_rates,
            "other_decode_layouts": dec_rates,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kv_append_attend_decode",
            "achieved": round(att_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(att_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
