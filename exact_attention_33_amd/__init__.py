"""Exact softmax attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libattn.so`` (hand-written gfx950
kernels behind a C ABI, declared in ``include/attn.h``).  ``ops`` is a thin
ctypes binding with the same entry-point names; it raises if the library is
missing -- there is no CPU fallback.
"""

__all__ = ["ops", "synth"]
