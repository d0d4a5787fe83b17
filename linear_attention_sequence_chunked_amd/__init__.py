"""Chunkwise gated-delta rule (forward, backward, decode step) for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/gdn.h`` (``libgdn.so``); :mod:`.gdn` is the thin ctypes binding.
"""
from .gdn import (bwd_workspace_size, chunk_bwd, chunk_fwd, chunk_fwd_segmented,  # noqa: F401
                  chunk_fwd_segmented_noalloc, chunk_fwd_varlen, decode_step, load_library,
                  segmented_workspace_size, segments_hint, status_string)

__all__ = ["chunk_fwd", "chunk_fwd_varlen", "chunk_fwd_segmented", "segmented_workspace_size",
           "segments_hint", "chunk_fwd_segmented_noalloc",
           "chunk_bwd", "bwd_workspace_size", "decode_step", "load_library", "status_string"]
