"""Comparison helpers for the GPU parity tests.

Relative L2 is ||x - ref||_2 / ||ref||_2 in float64.  Besides the figure over a
whole tensor, every test also bounds the worst LOCAL figure, so that one wrong
chunk of one stream cannot hide inside a large tensor:

- token tensors [B, T, H, ...] (o, dq, dk, dv): every (b, h, 64-token block);
- state tensors [B, H, V, K] (final state, d_initial_state): every (b, h);
- gate tensors [B, T, H] (dalpha, dbeta): every (b, h) over all tokens.

A block whose reference is exactly zero reports the absolute norm of the GPU
block instead (so an exact zero is required to pass a tolerance of 0).  A block
of fewer than MIN_BLOCK reference elements (a gate gradient of a stream shorter
than that) is left to the whole-tensor figure: its relative L2 is a
per-element relative error, which rounding of a cancelling dot product does not
bound, whatever the precision.
"""
from __future__ import annotations

import numpy as np

TBLOCK = 64
MIN_BLOCK = 16


def as_f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def rel_l2(x, ref):
    x, ref = as_f64(x), as_f64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _ratio(num2, den2):
    num, den = np.sqrt(num2), np.sqrt(den2)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def token_block_errors(x, ref, tblock: int = TBLOCK):
    """[B, T, H, ...] -> relative L2 of every (b, token block, h), shape [B, nb, H]."""
    x, ref = as_f64(x), as_f64(ref)
    B, T, H = ref.shape[:3]
    d2 = ((x - ref) ** 2).reshape(B, T, H, -1).sum(-1)
    r2 = (ref ** 2).reshape(B, T, H, -1).sum(-1)
    nb = -(-T // tblock)
    pad = nb * tblock - T
    if pad:
        d2 = np.concatenate([d2, np.zeros((B, pad, H))], axis=1)
        r2 = np.concatenate([r2, np.zeros((B, pad, H))], axis=1)
    d2 = d2.reshape(B, nb, tblock, H).sum(2)
    r2 = r2.reshape(B, nb, tblock, H).sum(2)
    return _ratio(d2, r2)


def stream_errors(x, ref, kind: str):
    """Relative L2 of every (b, h): kind 'state' for [B,H,V,K], 'gate' for [B,T,H]."""
    x, ref = as_f64(x), as_f64(ref)
    if kind == "state":
        B, H = ref.shape[:2]
        d2 = ((x - ref) ** 2).reshape(B, H, -1).sum(-1)
        r2 = (ref ** 2).reshape(B, H, -1).sum(-1)
    elif kind == "gate":
        d2 = ((x - ref) ** 2).sum(1)
        r2 = (ref ** 2).sum(1)
    else:
        raise ValueError(kind)
    return _ratio(d2, r2)


KIND = {"o": "token", "dq": "token", "dk": "token", "dv": "token",
        "final_state": "state", "d_initial_state": "state",
        "dalpha": "gate", "dbeta": "gate"}


def local_errors(name: str, x, ref):
    kind = KIND[name]
    if kind == "token":
        return token_block_errors(x, ref)
    if kind == "gate" and as_f64(ref).shape[1] < MIN_BLOCK:
        return np.zeros((0,))
    return stream_errors(x, ref, kind)


def worst_local(name: str, x, ref):
    """(worst local relative L2, index of that block) for a named tensor."""
    e = local_errors(name, x, ref)
    if e.size == 0:
        return 0.0, ()
    i = np.unravel_index(int(np.argmax(e)), e.shape)
    return float(e[i]), tuple(int(j) for j in i)


def assert_parity(label: str, tensors: dict, tol: float, local_tol: float | None = None):
    """tensors: name -> (gpu tensor, float64 reference).  Asserts the whole-tensor
    and the worst local relative L2 of each against tol (local_tol if given) and
    prints both, with the index of the worst block."""
    local_tol = tol if local_tol is None else local_tol
    msgs, fails = [], []
    for name, (x, ref) in tensors.items():
        e = rel_l2(x, ref)
        w, at = worst_local(name, x, ref)
        msgs.append("%s=%.2e (worst block %.2e at %s)" % (name, e, w, at))
        if not (np.isfinite(e) and e <= tol):
            fails.append((name, "whole", e))
        if not (np.isfinite(w) and w <= local_tol):
            fails.append((name, "block", w, at))
    print("  " + "; ".join(msgs), flush=True)
    assert not fails, (label, fails)
