"""Chunkwise gated-delta-rule forward for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/gdn.h`` (``libgdn.so``); :mod:`.gdn` is the thin ctypes binding.
"""
from .gdn import chunk_fwd, load_library, status_string  # noqa: F401

__all__ = ["chunk_fwd", "load_library", "status_string"]
