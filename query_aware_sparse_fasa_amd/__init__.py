"""FASA decode hot path (TIP -> per-kv-head top-B -> FAC) for MI355X / gfx950.

The compute runs in hand-written HIP kernels behind the C-ABI library
``libfasa.so`` (declared in include/fasa.h).  ``query_aware_sparse_fasa_amd.fasa``
is the thin ctypes binding; it loads the library on first use and raises if it
is missing -- there is no CPU fallback.
"""
__all__ = ["synth", "costmodel"]
