"""CPU oracle for the transform-coded KV cache and decode attention over it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its Python binding; the only module both sides import is
``workloads`` (seeded synthetic inputs, no codec arithmetic).

Everything is plain numpy in float64, written from the definitions on the
pages (cited per function) so that it can be checked by eye:

* ``transform``  -- Sylvester Hadamard, random-sign fold, data-derived basis, KL/MSE weights
* ``quantizer``  -- per-token fp16 min/step uniform b-bit quantizer, dequantizer, q(b)
* ``packing``    -- fixed-width little-endian bit packing of records
* ``codec``      -- project -> quantize -> pack, cache layout
* ``attention``  -- decode attention over the dequantized cache, textbook attention
* ``rope``       -- rotary position embedding; attention over keys compressed before it
* ``allocation`` -- rate-distortion model D(r, b) and the per-head C1 rank/bit search

Pinned by the ``-m "not gpu"`` tests against closed forms, hand-worked
examples (``tests/golden``), brute force and textbook special cases.  No
function here is "parity unpinned".
"""
from . import allocation, attention, codec, packing, quantizer, rope, transform, vq  # noqa: F401
