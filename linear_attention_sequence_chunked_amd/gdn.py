"""Python binding of libgdn (ctypes).  Argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI declared
in ``include/gdn.h``; this module checks tensors, allocates outputs with torch
(device memory and streams are all torch is used for), and forwards raw device
pointers plus the HIP stream (torch's current one unless ``stream=`` is given;
memory the binding allocates for a call on another stream is recorded on that
stream, so the caching allocator does not reuse it while the call still runs).  If the built library is missing it raises
at load time: there is no CPU or PyTorch fallback.

Operator contract ("OpenGDN 0.1.0", section "Core operator reference"): q, k
[B,T,H,K], v [B,T,H,V], alpha, beta [B,T,H], state [B,H,V,K]; feeding the
returned final state back as ``initial_state`` continues the stream exactly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_SUCCESS = 0
GDN_ERROR_INVALID_VALUE = 1
GDN_ERROR_NOT_SUPPORTED = 2
GDN_ERROR_LAUNCH = 3
GDN_ERROR_SCRATCH_LIMIT = 4
SEGMENTED_NOALLOC_MAX_BYTES = 64 << 20
GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

_DTYPES = {torch.float32: GDN_DTYPE_F32, torch.bfloat16: GDN_DTYPE_BF16}

# every symbol the header declares, with its ctypes signature
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "gdn_abi_version": (ctypes.c_int, []),
    "gdn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdn_chunk_fwd": (ctypes.c_int, [_VP] * 8 + [_I64] * 6 + [ctypes.c_int, _VP]),
    "gdn_chunk_fwd_varlen": (ctypes.c_int, [_VP] * 6 + [_I64] + [_VP] * 3 + [_I64] * 5 +
                             [ctypes.c_int, _VP]),
    "gdn_chunk_fwd_segments_hint": (ctypes.c_int64, [_I64] * 7),
    "gdn_chunk_fwd_segmented_workspace_size": (ctypes.c_size_t, [_I64] * 7),
    "gdn_chunk_fwd_segmented": (ctypes.c_int, [_VP] * 8 + [_I64] * 7 + [_VP, ctypes.c_size_t] +
                                [ctypes.c_int, _VP]),
    "gdn_chunk_fwd_segmented_noalloc": (ctypes.c_int, [_VP] * 8 + [_I64] * 7 + [ctypes.c_int, _VP]),
    "gdn_decode_step": (ctypes.c_int, [_VP] * 7 + [_I64] * 4 + [ctypes.c_int, _VP]),
    "gdn_chunk_bwd_workspace_size": (ctypes.c_size_t, [_I64] * 6 + [ctypes.c_int]),
    "gdn_chunk_bwd": (ctypes.c_int, [_VP] * 15 + [ctypes.c_size_t] + [_I64] * 6 + [ctypes.c_int, _VP]),
}

_lib = None


class GdnError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load libgdn.so (built ahead of time by ``build.build()``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(
                "libgdn.so is not built (%s); run __graft_entry__.build() or "
                "python -m linear_attention_sequence_chunked_amd.build" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load_library().gdn_status_string(int(code)).decode()


def _raise_for(code: int, what: str):
    if code == GDN_SUCCESS:
        return
    msg = "%s: %s" % (what, status_string(code))
    if code == GDN_ERROR_INVALID_VALUE:
        raise ValueError(msg)
    if code == GDN_ERROR_NOT_SUPPORTED:
        raise NotImplementedError(msg)
    raise GdnError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _launch_stream(dev, stream):
    """The stream a call enqueues on (``stream``, else torch's current stream of
    ``dev``) and whether it differs from torch's current stream."""
    cur = torch.cuda.current_stream(dev)
    s = stream if stream is not None else cur
    return s, s.cuda_stream != cur.cuda_stream


def _keep_for(s, other, tensors):
    """Tensors this binding allocated on torch's current stream but handed to work
    on another stream ``s``: tell the caching allocator, so that none of their
    memory is given to new work on the current stream before ``s`` is done with
    it (a scratch buffer is freed as soon as the call returns)."""
    if other:
        for t in tensors:
            if t is not None:
                t.record_stream(s)


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def chunk_fwd(q, k, v, alpha, beta, initial_state=None, chunk: int = 64, *,
              out=None, final_state=None, want_final_state: bool = True, stream=None):
    """Gated-delta-rule forward through ``gdn_chunk_fwd``.

    Returns ``(o, final_state)``; ``final_state`` is None when
    ``want_final_state`` is False.  ``final_state`` may be passed as the same
    tensor as ``initial_state`` to advance the state in place.  The call is
    asynchronous on ``stream`` (default: torch's current stream of q's device).
    """
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B,T,H,K]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    if q.dtype not in _DTYPES:
        raise NotImplementedError("dtype %s is not supported (float32 or bfloat16)" % q.dtype)
    B, T, H, K = q.shape
    if v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B,T,H,V]")
    V = v.shape[-1]
    _check(k, "k", (B, T, H, K), q.dtype, dev)
    _check(v, "v", (B, T, H, V), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(q, "q", (B, T, H, K), q.dtype, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, V, K), torch.float32, dev)
    made = []
    if out is None:
        out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
        made.append(out)
    else:
        _check(out, "out", (B, T, H, V), q.dtype, dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, V, K), dtype=torch.float32, device=dev)
        made.append(final_state)
    elif final_state is not None:
        _check(final_state, "final_state", (B, H, V, K), torch.float32, dev)
    with torch.cuda.device(dev):
        s, other = _launch_stream(dev, stream)
        rc = lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(initial_state), _ptr(out), _ptr(final_state),
                               B, T, H, K, V, int(chunk), _DTYPES[q.dtype],
                               ctypes.c_void_p(s.cuda_stream))
    _raise_for(rc, "gdn_chunk_fwd")
    _keep_for(s, other, made)
    return out, final_state


def bwd_workspace_size(B: int, T: int, H: int, K: int, V: int, chunk: int = 64,
                       dtype=torch.bfloat16) -> int:
    """Bytes of device workspace ``gdn_chunk_bwd`` needs for these sizes and dtype."""
    if dtype not in _DTYPES:
        raise NotImplementedError("dtype %s is not supported (float32 or bfloat16)" % dtype)
    return int(load_library().gdn_chunk_bwd_workspace_size(B, T, H, K, V, chunk, _DTYPES[dtype]))


def chunk_bwd(q, k, v, alpha, beta, d_o, initial_state=None, d_final_state=None,
              chunk: int = 64, *, want_d_initial_state: bool = True, workspace=None,
              out=None, stream=None):
    """Reverse mode of :func:`chunk_fwd` through ``gdn_chunk_bwd`` for the loss
    ``<o, d_o> + <final_state, d_final_state>``.

    Returns ``(dq, dk, dv, dalpha, dbeta, d_initial_state)``; the last is None
    when ``want_d_initial_state`` is False.  ``workspace`` may be a preallocated
    uint8 device tensor of at least :func:`bwd_workspace_size` bytes; ``out`` may
    be a tuple of the six preallocated results (d_initial_state None to skip it),
    which are then written and returned.
    """
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B,T,H,K]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    if q.dtype not in _DTYPES:
        raise NotImplementedError("dtype %s is not supported (float32 or bfloat16)" % q.dtype)
    B, T, H, K = q.shape
    if v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B,T,H,V]")
    V = v.shape[-1]
    _check(q, "q", (B, T, H, K), q.dtype, dev)
    _check(k, "k", (B, T, H, K), q.dtype, dev)
    _check(v, "v", (B, T, H, V), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(d_o, "d_o", (B, T, H, V), q.dtype, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, V, K), torch.float32, dev)
    if d_final_state is not None:
        _check(d_final_state, "d_final_state", (B, H, V, K), torch.float32, dev)
    need = lib.gdn_chunk_bwd_workspace_size(B, T, H, K, V, int(chunk), _DTYPES[q.dtype])
    made = []
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=dev)
        made.append(workspace)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    if out is not None:
        if len(out) != 6:
            raise ValueError("out must hold (dq, dk, dv, dalpha, dbeta, d_initial_state)")
        dq, dk, dv, dalpha, dbeta, d_s0 = out
        _check(dq, "dq", (B, T, H, K), q.dtype, dev)
        _check(dk, "dk", (B, T, H, K), q.dtype, dev)
        _check(dv, "dv", (B, T, H, V), q.dtype, dev)
        _check(dalpha, "dalpha", (B, T, H), torch.float32, dev)
        _check(dbeta, "dbeta", (B, T, H), torch.float32, dev)
        if d_s0 is not None:
            _check(d_s0, "d_initial_state", (B, H, V, K), torch.float32, dev)
    else:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        dalpha = torch.empty_like(alpha)
        dbeta = torch.empty_like(beta)
        d_s0 = (torch.empty((B, H, V, K), dtype=torch.float32, device=dev)
                if want_d_initial_state else None)
        made += [dq, dk, dv, dalpha, dbeta, d_s0]
    with torch.cuda.device(dev):
        s, other = _launch_stream(dev, stream)
        rc = lib.gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(dalpha), _ptr(dbeta), _ptr(d_s0),
                               _ptr(workspace), workspace.numel(), B, T, H, K, V, int(chunk),
                               _DTYPES[q.dtype], ctypes.c_void_p(s.cuda_stream))
    _raise_for(rc, "gdn_chunk_bwd")
    _keep_for(s, other, made)
    return dq, dk, dv, dalpha, dbeta, d_s0


def decode_step(q, k, v, alpha, beta, state, *, out=None, stream=None):
    """One token through ``gdn_decode_step``: ``state`` [B,H,V,K] float32 is
    advanced in place and ``o`` [B,H,V] is returned.  q, k [B,H,K], v [B,H,V] in
    float32 or bfloat16, alpha and beta [B,H] float32."""
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [B,H,K]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    if q.dtype not in _DTYPES:
        raise NotImplementedError("dtype %s is not supported (float32 or bfloat16)" % q.dtype)
    B, H, K = q.shape
    if v.dim() != 3:
        raise ValueError("v must be a 3-D tensor [B,H,V]")
    V = v.shape[-1]
    _check(k, "k", (B, H, K), q.dtype, dev)
    _check(v, "v", (B, H, V), q.dtype, dev)
    _check(alpha, "alpha", (B, H), torch.float32, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    _check(state, "state", (B, H, V, K), torch.float32, dev)
    _check(q, "q", (B, H, K), q.dtype, dev)
    made = []
    if out is None:
        out = torch.empty((B, H, V), dtype=q.dtype, device=dev)
        made.append(out)
    else:
        _check(out, "out", (B, H, V), q.dtype, dev)
    with torch.cuda.device(dev):
        s, other = _launch_stream(dev, stream)
        rc = lib.gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state),
                                 _ptr(out), B, H, K, V, _DTYPES[q.dtype], ctypes.c_void_p(s.cuda_stream))
    _raise_for(rc, "gdn_decode_step")
    _keep_for(s, other, made)
    return out


def chunk_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, initial_state=None, chunk: int = 64, *,
                     out=None, final_state=None, want_final_state: bool = True, stream=None):
    """Packed variable-length forward through ``gdn_chunk_fwd_varlen``.

    q, k [1,T,H,K], v [1,T,H,V], alpha, beta [1,T,H] hold N sequences back to back;
    ``cu_seqlens`` is an int32 device tensor [N+1] of offsets (0 .. T).  States are
    [N,H,V,K].  Returns ``(o, final_state)``.
    """
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 4 or q.shape[0] != 1:
        raise ValueError("q must be a 4-D tensor [1,T,H,K] (sequences packed along T)")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    if q.dtype not in _DTYPES:
        raise NotImplementedError("dtype %s is not supported (float32 or bfloat16)" % q.dtype)
    _, T, H, K = q.shape
    if v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [1,T,H,V]")
    V = v.shape[-1]
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor [N+1]")
    N = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _check(k, "k", (1, T, H, K), q.dtype, dev)
    _check(v, "v", (1, T, H, V), q.dtype, dev)
    _check(alpha, "alpha", (1, T, H), torch.float32, dev)
    _check(beta, "beta", (1, T, H), torch.float32, dev)
    _check(q, "q", (1, T, H, K), q.dtype, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, V, K), torch.float32, dev)
    made = []
    if out is None:
        out = torch.empty((1, T, H, V), dtype=q.dtype, device=dev)
        made.append(out)
    else:
        _check(out, "out", (1, T, H, V), q.dtype, dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=dev)
        made.append(final_state)
    elif final_state is not None:
        _check(final_state, "final_state", (N, H, V, K), torch.float32, dev)
    with torch.cuda.device(dev):
        s, other = _launch_stream(dev, stream)
        rc = lib.gdn_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                      _ptr(cu_seqlens), N, _ptr(initial_state), _ptr(out),
                                      _ptr(final_state), T, H, K, V, int(chunk), _DTYPES[q.dtype],
                                      ctypes.c_void_p(s.cuda_stream))
    _raise_for(rc, "gdn_chunk_fwd_varlen")
    _keep_for(s, other, made)
    return out, final_state


def segments_hint(B: int, T: int, H: int, K: int, V: int, chunk: int = 64, num_cus: int = 0) -> int:
    """Segment count ``gdn_chunk_fwd_segments_hint`` suggests (1: the plain call);
    ``num_cus`` = 0 plans for the current device.  0 when a size is not positive."""
    return int(load_library().gdn_chunk_fwd_segments_hint(B, T, H, K, V, chunk, num_cus))


def segmented_workspace_size(B: int, T: int, H: int, K: int, V: int, chunk: int, segments: int) -> int:
    """Bytes of device workspace ``gdn_chunk_fwd_segmented`` needs."""
    return int(load_library().gdn_chunk_fwd_segmented_workspace_size(B, T, H, K, V, chunk, segments))


def chunk_fwd_segmented(q, k, v, alpha, beta, initial_state=None, chunk: int = 64,
                        segments=None, *, out=None, final_state=None,
                        want_final_state: bool = True, workspace=None, stream=None):
    """:func:`chunk_fwd` computed segment-parallel (``gdn_chunk_fwd_segmented``):
    each sequence is split into ``segments`` pieces processed in parallel, joined by
    their affine state maps (``None``: the count :func:`segments_hint` gives for the
    tensors' device).  Returns ``(o, final_state)``."""
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B,T,H,K]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    if q.dtype not in _DTYPES:
        raise NotImplementedError("dtype %s is not supported (float32 or bfloat16)" % q.dtype)
    B, T, H, K = q.shape
    if v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B,T,H,V]")
    V = v.shape[-1]
    _check(k, "k", (B, T, H, K), q.dtype, dev)
    _check(v, "v", (B, T, H, V), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, V, K), torch.float32, dev)
    made = []
    if out is None:
        out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
        made.append(out)
    else:
        _check(out, "out", (B, T, H, V), q.dtype, dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, V, K), dtype=torch.float32, device=dev)
        made.append(final_state)
    elif final_state is not None:
        _check(final_state, "final_state", (B, H, V, K), torch.float32, dev)
    if segments is None:
        with torch.cuda.device(dev):
            segments = max(1, int(lib.gdn_chunk_fwd_segments_hint(B, T, H, K, V, int(chunk), 0)))
    need = int(lib.gdn_chunk_fwd_segmented_workspace_size(B, T, H, K, V, int(chunk), int(segments)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        made.append(workspace)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    with torch.cuda.device(dev):
        s, other = _launch_stream(dev, stream)
        rc = lib.gdn_chunk_fwd_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                         _ptr(initial_state), _ptr(out), _ptr(final_state), B, T,
                                         H, K, V, int(chunk), int(segments), _ptr(workspace),
                                         workspace.numel(), _DTYPES[q.dtype],
                                         ctypes.c_void_p(s.cuda_stream))
    _raise_for(rc, "gdn_chunk_fwd_segmented")
    _keep_for(s, other, made)
    return out, final_state


def chunk_fwd_segmented_noalloc(q, k, v, alpha, beta, initial_state=None, chunk: int = 64,
                                segments: int = 4, *, out=None, final_state=None,
                                want_final_state: bool = True, stream=None):
    """:func:`chunk_fwd_segmented` through ``gdn_chunk_fwd_segmented_noalloc``: the
    library's static per-device scratch (``SEGMENTED_NOALLOC_MAX_BYTES``) replaces
    the workspace, so the library allocates nothing; calls that overlap in time on
    one device race on that scratch.  ``out`` and ``final_state`` may be passed in
    so that the call allocates nothing on the torch side either.  Returns
    ``(o, final_state)``; raises ``MemoryError`` when the call needs more scratch
    than the static buffer holds."""
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B,T,H,K]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    if q.dtype not in _DTYPES:
        raise NotImplementedError("dtype %s is not supported (float32 or bfloat16)" % q.dtype)
    B, T, H, K = q.shape
    if v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B,T,H,V]")
    V = v.shape[-1]
    _check(k, "k", (B, T, H, K), q.dtype, dev)
    _check(v, "v", (B, T, H, V), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, V, K), torch.float32, dev)
    made = []
    if out is None:
        out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
        made.append(out)
    else:
        _check(out, "out", (B, T, H, V), q.dtype, dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, V, K), dtype=torch.float32, device=dev)
        made.append(final_state)
    elif final_state is not None:
        _check(final_state, "final_state", (B, H, V, K), torch.float32, dev)
    with torch.cuda.device(dev):
        s, other = _launch_stream(dev, stream)
        rc = lib.gdn_chunk_fwd_segmented_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(out),
            _ptr(final_state), B, T, H, K, V, int(chunk), int(segments), _DTYPES[q.dtype],
            ctypes.c_void_p(s.cuda_stream))
    if rc == GDN_ERROR_SCRATCH_LIMIT:
        raise MemoryError("gdn_chunk_fwd_segmented_noalloc: %s" % status_string(rc))
    _raise_for(rc, "gdn_chunk_fwd_segmented_noalloc")
    _keep_for(s, other, made)
    return out, final_state
