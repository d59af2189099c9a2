"""decode_attention_04_amd -- transform-coded low-bit KV cache and decode attention over it, for MI355X.

* ``libkvtc.so`` (built from ``csrc/`` by ``python -m decode_attention_04_amd.build``):
  the C-ABI library of hand-written gfx950 kernels declared in ``include/kvtc.h``.
* ``_lib``: the thin ctypes binding with the same entry-point names.
* ``calib``: host-side calibration that produces the library's inputs (per-head
  basis with the random-sign Hadamard folded in, C1 rank/bit allocation).

The binding names below load the library on first use and raise ImportError if
it has not been built (there is no fallback implementation).
"""
_BINDING = (
    "KV_ERR_CAPACITY", "KV_ERR_DEVICE", "KV_ERR_INVALID", "KV_ERR_UNSUPPORTED", "KV_OK", "KvError",
    "Layout", "kv_append", "kv_append_attend_decode", "kv_append_attend_decode_noalloc", "kv_attend_decode", "kv_attend_plan", "kv_attend_decode_ragged", "kv_cache_bytes", "kv_decode", "kv_encode", "kv_quantize_pack",
    "kv_record_words", "kv_unpack", "kv_workspace_bytes",
    "kv_attend_decode_rope", "kv_append_attend_decode_rope", "kv_workspace_bytes_rope",
)


def __getattr__(name):
    if name in _BINDING:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)


__all__ = list(_BINDING)
