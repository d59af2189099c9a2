"""ctypes binding of libkvtc.so: argument marshalling only.

Every computation of the encode and decode path runs in the HIP kernels of
the library; this module converts tensors to device pointers, passes the
caller's current HIP stream and turns non-zero status codes into exceptions.
Importing it fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVTC_LIBRARY may name another build of the same library (the phase-stamp diagnostic
# variant libkvtc_stamps.so); by default the package's libkvtc.so.
LIB_PATH = os.environ.get("KVTC_LIBRARY") or os.path.join(_PKG, "libkvtc.so")

KV_OK, KV_ERR_INVALID, KV_ERR_UNSUPPORTED, KV_ERR_CAPACITY, KV_ERR_DEVICE = range(5)
KV_F32, KV_F16 = 0, 1

EXPORTED = (
    "kv_record_words", "kv_cache_bytes", "kv_workspace_bytes", "kv_workspace_bytes_split", "kv_attend_plan",
    "kv_encode", "kv_append", "kv_attend_decode", "kv_attend_decode_split",
    "kv_append_attend_decode", "kv_attend_decode_ragged", "kv_append_attend_decode_noalloc",
    "kv_decode", "kv_quantize_pack", "kv_unpack", "kv_last_error",
    "kv_workspace_bytes_rope", "kv_attend_decode_rope", "kv_append_attend_decode_rope",
)


class KvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvtc status {status}: {message}")
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("rank_k", ctypes.POINTER(ctypes.c_int32)),
        ("bits_k", ctypes.POINTER(ctypes.c_int32)),
        ("rank_v", ctypes.POINTER(ctypes.c_int32)),
        ("bits_v", ctypes.POINTER(ctypes.c_int32)),
        ("scale_k", ctypes.POINTER(ctypes.c_uint32)),
        ("scale_v", ctypes.POINTER(ctypes.c_uint32)),
        ("query_basis_k", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32),
        ("pool_pages", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("vq_k", ctypes.c_int32),
        ("vq_v", ctypes.c_int32),
        ("codebook_k", ctypes.c_void_p),
        ("codebook_v", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decode_attention_04_amd.build`")
    # PyTorch ships its own HIP runtime under the same soname.  Loading it first makes
    # the library bind to that runtime, so that both see the same devices, streams and
    # allocations (two HIP runtimes in one process do not share device state).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L = ctypes.POINTER(_Layout)
    sig = {
        "kv_record_words": (i32, [i32, i32]),
        "kv_cache_bytes": (i32, [L, i32, ctypes.POINTER(sz)]),
        "kv_workspace_bytes": (i32, [L, i64, ctypes.POINTER(sz)]),
        "kv_workspace_bytes_split": (i32, [L, i64, i64, ctypes.POINTER(sz)]),
        "kv_attend_plan": (i32, [L, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "kv_encode": (i32, [L, P, P, i32, i64, i64, P, P, P, P, P]),
        "kv_append": (i32, [L, P, P, i32, i64, P, P, P, P, P]),
        "kv_attend_decode": (i32, [L, P, i32, i64, P, P, P, P, f32, P, P, sz, P]),
        "kv_attend_decode_split": (i32, [L, P, i32, i64, i64, P, P, P, P, f32, P, P, sz, P]),
        "kv_append_attend_decode": (i32, [L, P, P, i32, P, i32, i64, i64, P, P, P, P, f32, P, P, sz, P]),
        "kv_attend_decode_ragged": (i32, [L, P, i32, P, i64, P, P, P, P, f32, P, P, sz, P]),
        "kv_append_attend_decode_noalloc": (i32, [L, P, P, i32, P, i32, i64, i64, P, P, P, P, f32, P, P]),
        "kv_decode": (i32, [L, i32, i64, i64, P, P, P, P]),
        "kv_workspace_bytes_rope": (i32, [L, i64, i64, ctypes.POINTER(sz)]),
        "kv_attend_decode_rope": (i32, [L, P, i32, i64, i64, P, P, P, P, f32, P, P, P, sz, P]),
        "kv_append_attend_decode_rope": (i32, [L, P, P, i32, P, i32, i64, i64, P, P, P, P, f32, P, P, P, sz, P]),
        "kv_quantize_pack": (i32, [P, i64, i32, i32, P, P]),
        "kv_unpack": (i32, [P, i64, i32, i32, P, P, P]),
        "kv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _check(status: int):
    if status != KV_OK:
        raise KvError(status, _lib.kv_last_error().decode())


class Layout:
    """Shape and per-head (rank, bits) allocation of one layer's compressed cache.

    ``alloc`` lists (rank_k, bits_k, rank_v, bits_v) per KV head.  ``scale_k`` /
    ``scale_v``: None (records with per-token headers) or one 32-bit word per KV
    head, the head's fixed quantizer for header-free records (fp16 bits of the min
    in bits 0-15, of the step in bits 16-31).  ``query_basis_k``: each head's key basis
    block holds the encode basis P_K then the query basis Q_K (a non-orthogonal key
    transform; keys are reconstructed as Q_K c^).  ``page_tokens`` > 0 makes the caches
    paged: each head's region is a pool of ``pool_pages`` pages and ``block_table`` (a
    device int32 tensor [batch, capacity // page_tokens]) maps each sequence's logical
    pages to pool pages.  ``codebook_k`` / ``codebook_v``: device uint32 (int32) tensors of
    per-pair codebooks make that tensor's records vector-quantized over coordinate pairs
    (the allocation's bits are then index bits per pair).
    """

    def __init__(self, n_kv_heads: int, n_q_heads: int, batch: int, capacity: int,
                 alloc: Sequence[Tuple[int, int, int, int]], head_dim: int = 128,
                 scale_k: Optional[Sequence[int]] = None, scale_v: Optional[Sequence[int]] = None,
                 query_basis_k: bool = False, page_tokens: int = 0, pool_pages: int = 0, block_table=None,
                 codebook_k=None, codebook_v=None):
        if len(alloc) != n_kv_heads:
            raise ValueError("alloc needs one (rank_k, bits_k, rank_v, bits_v) per KV head")
        self.head_dim, self.n_kv_heads, self.n_q_heads = head_dim, n_kv_heads, n_q_heads
        self.batch, self.capacity = batch, capacity
        self.alloc = [tuple(int(x) for x in a) for a in alloc]
        arr = ctypes.c_int32 * n_kv_heads
        self._rk = arr(*[a[0] for a in self.alloc])
        self._bk = arr(*[a[1] for a in self.alloc])
        self._rv = arr(*[a[2] for a in self.alloc])
        self._bv = arr(*[a[3] for a in self.alloc])
        u32 = ctypes.c_uint32 * n_kv_heads
        for name, sc in (("scale_k", scale_k), ("scale_v", scale_v)):
            if sc is not None and len(sc) != n_kv_heads:
                raise ValueError(f"{name} needs one word per KV head")
        self.scale_k = None if scale_k is None else [int(x) for x in scale_k]
        self.scale_v = None if scale_v is None else [int(x) for x in scale_v]
        self._sk = None if scale_k is None else u32(*self.scale_k)
        self._sv = None if scale_v is None else u32(*self.scale_v)
        self.query_basis_k = bool(query_basis_k)
        self._c = _Layout(head_dim, n_kv_heads, n_q_heads, batch, capacity,
                          self._rk, self._bk, self._rv, self._bv,
                          ctypes.cast(self._sk, ctypes.POINTER(ctypes.c_uint32)) if self._sk else None,
                          ctypes.cast(self._sv, ctypes.POINTER(ctypes.c_uint32)) if self._sv else None,
                          int(self.query_basis_k), int(page_tokens), int(pool_pages), _ptr(block_table) or None,
                          2 if codebook_k is not None else 0, 2 if codebook_v is not None else 0,
                          _ptr(codebook_k) or None, _ptr(codebook_v) or None)
        self.page_tokens, self.pool_pages = int(page_tokens), int(pool_pages)
        self.vq_k, self.vq_v = codebook_k is not None, codebook_v is not None
        # keep the device tensors alive while the layout is used
        self._block_table, self._codebooks = block_table, (codebook_k, codebook_v)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def ref(self):
        return ctypes.byref(self._c)


def _ptr(t) -> int:
    if t is None:
        return 0
    if hasattr(t, "is_cuda") and not t.is_cuda:
        raise ValueError("tensor must live in device memory")
    if hasattr(t, "is_contiguous") and not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return KV_F32
    if t.dtype == torch.float16:
        return KV_F16
    raise ValueError(f"unsupported dtype {t.dtype}")


def kv_record_words(rank: int, bits: int) -> int:
    return int(_lib.kv_record_words(rank, bits))


def kv_cache_bytes(layout: Layout, which: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.kv_cache_bytes(layout.ref(), which, ctypes.byref(out)))
    return out.value


def kv_workspace_bytes(layout: Layout, n_tokens: int, split_tokens: int = 0) -> int:
    out = ctypes.c_size_t()
    _check(_lib.kv_workspace_bytes_split(layout.ref(), n_tokens, split_tokens, ctypes.byref(out)))
    return out.value


def kv_attend_plan(layout: Layout, n_tokens: int, split_tokens: int = 0):
    """(kernel class, largest split count, grid size) of decode attention over `layout`:
    class -1 is the generic kernel, 0-5 the built-in budget classes, 6+ the frozen ones."""
    c, n, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.kv_attend_plan(layout.ref(), n_tokens, split_tokens, ctypes.byref(c), ctypes.byref(n),
                               ctypes.byref(w)))
    return c.value, n.value, w.value


def kv_encode(layout, k, v, n_tokens, pos0, basis_k, basis_v, cache_k, cache_v, stream=None):
    """Prefill encode of k, v [batch, n_kv_heads, n_tokens, head_dim] (float32 or float16)."""
    _check(_lib.kv_encode(layout.ref(), _ptr(k), _ptr(v), _dtype_code(k), n_tokens, pos0,
                          _ptr(basis_k), _ptr(basis_v), _ptr(cache_k), _ptr(cache_v), _stream(stream)))


def kv_append(layout, k1, v1, pos, basis_k, basis_v, cache_k, cache_v, stream=None):
    """Append one token per (sequence, head): k1, v1 [batch, n_kv_heads, head_dim]."""
    _check(_lib.kv_append(layout.ref(), _ptr(k1), _ptr(v1), _dtype_code(k1), pos,
                          _ptr(basis_k), _ptr(basis_v), _ptr(cache_k), _ptr(cache_v), _stream(stream)))


def kv_attend_decode(layout, q, n_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale, out,
                     workspace, split_tokens: int = 0, stream=None):
    """Decode attention: q [batch, n_q_heads, head_dim] -> out (float32, same shape).

    ``workspace`` holds at least kv_workspace_bytes(layout, n_tokens, split_tokens)
    bytes and starts zero-filled (torch.zeros); calls leave its counter words zero.
    """
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.kv_attend_decode_split(layout.ref(), _ptr(q), _dtype_code(q), n_tokens, split_tokens,
                                       _ptr(basis_k), _ptr(basis_v), _ptr(cache_k), _ptr(cache_v),
                                       float(softmax_scale), _ptr(out), _ptr(workspace), nbytes,
                                       _stream(stream)))


def kv_attend_decode_ragged(layout, q, lengths, max_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale,
                            out, workspace, stream=None):
    """Decode attention with per-sequence lengths: lengths is a device int32 tensor
    [batch] (sequence b attends over its tokens 0 .. lengths[b]-1, clamped to
    [0, max_tokens]); workspace as for kv_attend_decode at max_tokens."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.kv_attend_decode_ragged(layout.ref(), _ptr(q), _dtype_code(q), _ptr(lengths), max_tokens,
                                        _ptr(basis_k), _ptr(basis_v), _ptr(cache_k), _ptr(cache_v),
                                        float(softmax_scale), _ptr(out), _ptr(workspace), nbytes,
                                        _stream(stream)))


def kv_append_attend_decode(layout, k1, v1, q, n_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale,
                            out, workspace, split_tokens: int = 0, stream=None):
    """Append k1, v1 [batch, n_kv_heads, head_dim] at position n_tokens - 1 and attend
    over tokens 0 .. n_tokens-1 in one launch (workspace as for kv_attend_decode)."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.kv_append_attend_decode(layout.ref(), _ptr(k1), _ptr(v1), _dtype_code(k1), _ptr(q),
                                        _dtype_code(q), n_tokens, split_tokens, _ptr(basis_k), _ptr(basis_v),
                                        _ptr(cache_k), _ptr(cache_v), float(softmax_scale), _ptr(out),
                                        _ptr(workspace), nbytes, _stream(stream)))


def kv_append_attend_decode_noalloc(layout, k1, v1, q, n_tokens, basis_k, basis_v, cache_k, cache_v,
                                    softmax_scale, out, split_tokens: int = 0, stream=None):
    """kv_append_attend_decode with the split scratch in the library's static device
    array (no workspace argument; calls on one GPU must not overlap)."""
    _check(_lib.kv_append_attend_decode_noalloc(layout.ref(), _ptr(k1), _ptr(v1), _dtype_code(k1), _ptr(q),
                                                _dtype_code(q), n_tokens, split_tokens, _ptr(basis_k),
                                                _ptr(basis_v), _ptr(cache_k), _ptr(cache_v), float(softmax_scale),
                                                _ptr(out), _stream(stream)))


def kv_workspace_bytes_rope(layout: Layout, n_tokens: int, split_tokens: int = 0) -> int:
    """Workspace bytes of kv_attend_decode_rope (its own split plan)."""
    out = ctypes.c_size_t()
    _check(_lib.kv_workspace_bytes_rope(layout.ref(), n_tokens, split_tokens, ctypes.byref(out)))
    return out.value


def kv_attend_decode_rope(layout, q, n_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale, inv_freq, out,
                          workspace, split_tokens: int = 0, stream=None):
    """Decode attention over keys compressed before RoPE: q [batch, n_q_heads, head_dim]
    (already rotated to its position), inv_freq a device float64 tensor [head_dim / 2];
    token t's key is turned by t * inv_freq.  Workspace: kv_workspace_bytes_rope bytes,
    zero-filled on first use."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.kv_attend_decode_rope(layout.ref(), _ptr(q), _dtype_code(q), n_tokens, split_tokens,
                                      _ptr(basis_k), _ptr(basis_v), _ptr(cache_k), _ptr(cache_v),
                                      float(softmax_scale), _ptr(inv_freq), _ptr(out), _ptr(workspace), nbytes,
                                      _stream(stream)))


def kv_append_attend_decode_rope(layout, k1, v1, q, n_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale,
                                 inv_freq, out, workspace, split_tokens: int = 0, stream=None):
    """Append the unrotated k1, v1 at position n_tokens - 1, then attend as
    kv_attend_decode_rope, in one launch."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.kv_append_attend_decode_rope(layout.ref(), _ptr(k1), _ptr(v1), _dtype_code(k1), _ptr(q),
                                             _dtype_code(q), n_tokens, split_tokens, _ptr(basis_k), _ptr(basis_v),
                                             _ptr(cache_k), _ptr(cache_v), float(softmax_scale), _ptr(inv_freq),
                                             _ptr(out), _ptr(workspace), nbytes, _stream(stream)))


def kv_decode(layout, which, n_tokens, pos0, basis, cache, out, stream=None):
    """Reconstruct records pos0 .. pos0+n_tokens-1 of tensor `which` (0 = K, 1 = V):
    out float32 [batch, n_kv_heads, n_tokens, head_dim] = P (min + step * code)."""
    _check(_lib.kv_decode(layout.ref(), which, n_tokens, pos0, _ptr(basis), _ptr(cache), _ptr(out),
                          _stream(stream)))


def kv_quantize_pack(coords, rank, bits, records, stream=None):
    """coords float32 [n, rank] -> records uint32/int32 [n, W]."""
    n = coords.shape[0] if coords.dim() > 1 else 0
    _check(_lib.kv_quantize_pack(_ptr(coords), n, rank, bits, _ptr(records), _stream(stream)))


def kv_unpack(records, n, rank, bits, min_step, codes, stream=None):
    """records [n, W] -> min_step int16/uint16 [n, 2] (fp16 bits) and codes uint8 [n, rank]."""
    _check(_lib.kv_unpack(_ptr(records), n, rank, bits, _ptr(min_step), _ptr(codes), _stream(stream)))


def raw():
    """The underlying ctypes library handle (for ABI tests)."""
    return _lib
