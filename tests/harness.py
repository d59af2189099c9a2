"""Shared test helpers: oracle-side calibration and caches, device transfers.

Expected values always come from ``oracle`` (CPU, float64); the GPU path only
ever receives the same inputs.
"""
from __future__ import annotations

import numpy as np

import workloads as W
from oracle import allocation, codec, transform

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


def oracle_cache(wl, alloc, bases_k, bases_v, batch, capacity, T, kv=None):
    """Flat K and V caches (uint32) holding the oracle's records of tokens 0..T-1.

    kv: optional dict (tensor, b, h) -> token array [T, d] (defaults to the workload's tokens).
    """
    rk = [a[0] for a in alloc]
    bk = [a[1] for a in alloc]
    rv = [a[2] for a in alloc]
    bv = [a[3] for a in alloc]
    ck = np.zeros(codec.region_offsets(rk, bk, batch, capacity)[-1], np.uint32)
    cv = np.zeros(codec.region_offsets(rv, bv, batch, capacity)[-1], np.uint32)
    for h in range(len(alloc)):
        for b in range(batch):
            xk = kv[("K", b, h)] if kv else W.tokens(wl, "K", b, h, 0, T)
            xv = kv[("V", b, h)] if kv else W.tokens(wl, "V", b, h, 0, T)
            s0, s1, _ = codec.record_slice(rk, bk, batch, capacity, h, b, 0, T)
            ck[s0:s1] = codec.encode_tokens(xk, bases_k[h], bk[h]).reshape(-1)
            s0, s1, _ = codec.record_slice(rv, bv, batch, capacity, h, b, 0, T)
            cv[s0:s1] = codec.encode_tokens(xv, bases_v[h], bv[h]).reshape(-1)
    return ck, cv


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
