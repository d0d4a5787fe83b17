"""Seeded synthetic inputs for the gated-delta-rule chunk forward.

This module draws random inputs and nothing else: it holds none of the
recurrence's arithmetic, so both the HIP path's tests/benchmark and the fp64
oracle can take their inputs from it.

Shapes follow the operator contract of "OpenGDN 0.1.0" (section "Core operator
reference"): q, k [B,T,H,K], v [B,T,H,V], alpha, beta [B,T,H], state [B,H,V,K].
Distributions follow the workloads the pages describe: q and k are L2-normalised
over the key axis (the mixer of "OpenGDN 0.1.0", section "Mixer"), beta is a
sigmoid, and alpha is either a sigmoid (OpenGDN's documented default) or the
decay exp(-0.1 * softplus(x)), a Mamba2-style log-gate of the kind "Sparse Delta
Memory: layer and kernels" uses in "What the layer computes".

All draws are made on the CPU with ``torch.Generator().manual_seed(seed)`` in
float32, in a fixed order (q, k, v, alpha logits, beta logits, then the initial
state and the output gradient when requested); q, k, v are then rounded to the
requested dtype, so every consumer sees identical values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    K: int
    V: int
    chunk: int
    dtype: torch.dtype
    gate: str               # "sigmoid" or "decay"
    s0_std: float | None = None
    with_do: bool = False
    split_at: int | None = None  # streaming seam for the long-context case
    seed: int = 0
    note: str = field(default="", compare=False)


# The five workloads of the operator (seeds equal the workload number), plus a decode
# batch (seed 6) and a few-stream long context (seed 9).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 64, 2, 16, 16, 16, torch.float32, "sigmoid", seed=1,
                          note="tiny fp32, B1 T64 H2 K=V=16, chunk 16"),
    "mid_bf16": Workload("mid_bf16", 2, 2048, 4, 128, 128, 64, torch.bfloat16, "decay", seed=2,
                         note="mid bf16 forward, B2 T2048 H4 K=V=128, chunk 64"),
    "train_bf16": Workload("train_bf16", 8, 4096, 6, 128, 128, 64, torch.bfloat16, "decay", seed=3,
                           note="training-shape forward, B8 T4096 H6 K=V=128, chunk 64"),
    "train_f32": Workload("train_f32", 8, 4096, 6, 128, 128, 64, torch.float32, "decay", seed=3,
                          note="training-shape forward with float32 q, k, v, o, B8 T4096 H6 "
                               "K=V=128, chunk 64"),
    "fwdbwd_bf16": Workload("fwdbwd_bf16", 4, 2048, 6, 128, 128, 64, torch.bfloat16, "decay",
                            with_do=True, seed=4,
                            note="forward+backward shape, B4 T2048 H6 K=V=128, chunk 64"),
    "fwdbwd_f32": Workload("fwdbwd_f32", 4, 2048, 6, 128, 128, 64, torch.float32, "decay",
                           with_do=True, seed=4,
                           note="forward+backward shape with float32 q, k, v, d_o, B4 T2048 H6 "
                                "K=V=128, chunk 64"),
    "long_few_bf16": Workload("long_few_bf16", 1, 32768, 2, 128, 128, 64, torch.bfloat16, "decay",
                              s0_std=0.02, seed=9,
                              note="long context with few streams, B1 T32768 H2 K=V=128, chunk 64 "
                                   "(the case segment parallelism is for)"),
    "decode_bf16": Workload("decode_bf16", 64, 1, 16, 128, 128, 64, torch.bfloat16, "decay",
                            s0_std=0.02, seed=6,
                            note="decode step, 64 streams x 16 heads, K=V=128, one token per "
                                 "call, S0 ~ 0.02 N(0,1)"),
    "long_bf16": Workload("long_bf16", 1, 32768, 16, 128, 128, 64, torch.bfloat16, "decay",
                          s0_std=0.02, split_at=16384, seed=5,
                          note="long-context streaming prefill, B1 T32768 H16 K=V=128, "
                               "chunk 64, S0 ~ 0.02 N(0,1), two 16384-token calls"),
}


def make_inputs(B: int, T: int, H: int, K: int, V: int, dtype=torch.bfloat16,
                seed: int = 0, gate: str = "decay", s0_std: float | None = None,
                with_do: bool = False, keys: str = "unit", beta_range=None) -> dict:
    """Draw one seeded input set on the CPU.

    Returns a dict with q, k, v (``dtype``), alpha, beta (float32 [B,T,H]),
    initial_state (float32 [B,H,V,K] or None) and d_o (``dtype`` or None).

    Edge-case options (drawn after every standard draw, so the standard inputs of
    a seed do not change):
      gate="strong"          alpha in (0.005, 0.2): the decay over a 64-token
                             chunk reaches about 2^-210, far below float32's range;
      gate="extreme"         alpha in (2^-16, 2^-4): the same for 16-token chunks;
      keys="correlated"      k_t = normalise(kbar + 0.1 n_t / sqrt(K)) with one
                             unit kbar per (batch, head): k_r . k_i ~ 0.99, so
                             I + tril(beta A, -1) is far from the identity;
      keys="repeated"        runs of 8 identical keys;
      beta_range=(lo, hi)    beta = lo + (hi - lo) sigmoid(x) instead of sigmoid(x).
    """
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn(B, T, H, K, generator=g, dtype=torch.float32)
    k = torch.randn(B, T, H, K, generator=g, dtype=torch.float32)
    v = torch.randn(B, T, H, V, generator=g, dtype=torch.float32)
    a_logit = torch.randn(B, T, H, generator=g, dtype=torch.float32)
    b_logit = torch.randn(B, T, H, generator=g, dtype=torch.float32)
    s0 = None
    if s0_std is not None:
        s0 = torch.randn(B, H, V, K, generator=g, dtype=torch.float32) * float(s0_std)
    d_o = None
    if with_do:
        d_o = torch.randn(B, T, H, V, generator=g, dtype=torch.float32).to(dtype)
    # unit-norm queries and keys along the key axis, normalised in float32
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    if keys == "correlated":
        kbar = torch.randn(B, 1, H, K, generator=g, dtype=torch.float32)
        kbar = kbar / kbar.norm(dim=-1, keepdim=True)
        noise = torch.randn(B, T, H, K, generator=g, dtype=torch.float32)
        k = kbar + (0.1 / K ** 0.5) * noise
        k = k / k.norm(dim=-1, keepdim=True)
    elif keys == "repeated":
        idx = (torch.arange(T) // 8) * 8
        k = k[:, idx].contiguous()
    elif keys != "unit":
        raise ValueError("keys must be 'unit', 'correlated' or 'repeated'")
    if gate == "sigmoid":
        alpha = torch.sigmoid(a_logit)
    elif gate == "decay":
        alpha = torch.exp(-0.1 * torch.nn.functional.softplus(a_logit))
    elif gate == "strong":
        alpha = 0.005 + 0.195 * torch.sigmoid(a_logit)
    elif gate == "extreme":
        alpha = torch.exp2(-(4.0 + 12.0 * torch.sigmoid(a_logit)))
    else:
        raise ValueError("gate must be 'sigmoid', 'decay', 'strong' or 'extreme'")
    beta = torch.sigmoid(b_logit)
    if beta_range is not None:
        lo, hi = beta_range
        beta = lo + (hi - lo) * beta
    return {
        "q": q.to(dtype).contiguous(), "k": k.to(dtype).contiguous(), "v": v.to(dtype).contiguous(),
        "alpha": alpha.contiguous(), "beta": beta.contiguous(),
        "initial_state": None if s0 is None else s0.contiguous(),
        "d_o": d_o,
    }


def workload_inputs(w: Workload | str, **overrides) -> dict:
    """Inputs of a named workload (overrides may shrink T or B for sampled checks)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    p = dict(B=w.B, T=w.T, H=w.H, K=w.K, V=w.V, dtype=w.dtype, seed=w.seed, gate=w.gate,
             s0_std=w.s0_std, with_do=w.with_do)
    p.update(overrides)
    return make_inputs(**p)


def make_inputs_on_device(B: int, T: int, H: int, K: int, V: int, device, dtype=torch.bfloat16,
                          seed: int = 0, gate: str = "decay", slab_tokens: int = 1 << 16) -> dict:
    """Draw a seeded input set directly in device memory, for sizes whose float32
    draws would not fit the host comfortably (gigabytes per token tensor).

    The same distributions as make_inputs (unit-norm q and k normalised in
    float32, decay or sigmoid alpha, sigmoid beta, no initial state), drawn with a
    device generator slab by slab along the token axis, so the float32 scratch
    stays at one slab.  The values differ from make_inputs' for the same seed;
    whoever checks them copies the tensors it needs back to the host.
    """
    g = torch.Generator(device=device).manual_seed(int(seed))
    q = torch.empty(B, T, H, K, dtype=dtype, device=device)
    k = torch.empty(B, T, H, K, dtype=dtype, device=device)
    v = torch.empty(B, T, H, V, dtype=dtype, device=device)
    for t0 in range(0, T, slab_tokens):
        t1 = min(T, t0 + slab_tokens)
        for dst, d in ((q, K), (k, K)):
            x = torch.randn(B, t1 - t0, H, d, generator=g, dtype=torch.float32, device=device)
            dst[:, t0:t1] = (x / x.norm(dim=-1, keepdim=True)).to(dtype)
        v[:, t0:t1] = torch.randn(B, t1 - t0, H, V, generator=g, dtype=torch.float32,
                                  device=device).to(dtype)
    a_logit = torch.randn(B, T, H, generator=g, dtype=torch.float32, device=device)
    b_logit = torch.randn(B, T, H, generator=g, dtype=torch.float32, device=device)
    if gate == "sigmoid":
        alpha = torch.sigmoid(a_logit)
    elif gate == "decay":
        alpha = torch.exp(-0.1 * torch.nn.functional.softplus(a_logit))
    else:
        raise ValueError("gate must be 'sigmoid' or 'decay'")
    return {"q": q, "k": k, "v": v, "alpha": alpha.contiguous(),
            "beta": torch.sigmoid(b_logit).contiguous(), "initial_state": None, "d_o": None}
