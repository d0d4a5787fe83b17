"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here.

The arithmetic lives in ``gdn_oracle.c`` (plain C, IEEE double, token by token);
this module compiles it with gcc and wraps it with ctypes over numpy float64
arrays.  See the header of ``gdn_oracle.c`` for the recurrence and its sources:
"Sparse Delta Memory: layer and kernels" (section "What the layer computes" and
the dense-limit paragraph of "Product-key top-k") and "OpenGDN 0.1.0"
(section "Core operator reference").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so next to it (portable -O2 x86-64)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [_D] * 8 + [_I64] * 5 + [ctypes.c_int]
        lib.gdn_oracle_bwd.restype = ctypes.c_int
        lib.gdn_oracle_bwd.argtypes = [_D] * 14 + [_I64] * 5 + [ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU); exact widening to float64
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


def fwd(q, k, v, alpha, beta, initial_state=None, nthreads: int | None = None):
    """Token-serial forward.  Returns (o [B,T,H,V], final_state [B,H,V,K]) as float64.

    q, k: [B,T,H,K]; v: [B,T,H,V]; alpha, beta: [B,T,H]; initial_state: [B,H,V,K]
    or None (zeros).  Inputs may be numpy arrays or CPU torch tensors of any float
    dtype: they are widened to float64 exactly.
    """
    q, k, v, alpha, beta, s0 = (_f64(x) for x in (q, k, v, alpha, beta, initial_state))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and v.shape == (B, T, H, V)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    if s0 is not None:
        assert s0.shape == (B, H, V, K)
    o = np.zeros((B, T, H, V), dtype=np.float64)
    sf = np.zeros((B, H, V, K), dtype=np.float64)
    rc = _load().gdn_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0),
                                _ptr(o), _ptr(sf), B, T, H, K, V,
                                int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("gdn_oracle_fwd failed with code %d" % rc)
    return o, sf


def bwd(q, k, v, alpha, beta, d_o, initial_state=None, d_final_state=None,
        nthreads: int | None = None):
    """Reverse mode of :func:`fwd` for the loss <o, d_o> + <final_state, d_final_state>.

    Returns a dict with dq, dk, dv, dalpha, dbeta, d_initial_state (float64).
    """
    q, k, v, alpha, beta, s0, do, dsf = (
        _f64(x) for x in (q, k, v, alpha, beta, initial_state, d_o, d_final_state))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert do.shape == (B, T, H, V)
    out = {
        "dq": np.zeros((B, T, H, K)), "dk": np.zeros((B, T, H, K)), "dv": np.zeros((B, T, H, V)),
        "dalpha": np.zeros((B, T, H)), "dbeta": np.zeros((B, T, H)),
        "d_initial_state": np.zeros((B, H, V, K)),
    }
    rc = _load().gdn_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0),
                                _ptr(do), _ptr(dsf), _ptr(out["dq"]), _ptr(out["dk"]),
                                _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]),
                                _ptr(out["d_initial_state"]), B, T, H, K, V,
                                int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("gdn_oracle_bwd failed with code %d" % rc)
    return out
