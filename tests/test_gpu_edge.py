"""Edge cases of the method on every entry point, against the fp64 oracle.

- Strong decay.  With alpha in (0.005, 0.2) the log-gate falls by up to 7.6
  (base 2) per token, so over a 64-token chunk the decay 2^(g_r - g_i) spans
  2^-490 .. 1 for i <= r, and the masked entries (i > r) have exponents up to
  +490: exponentiating before masking gives inf, and inf * 0 gives NaN.  The
  chunk algebra only ever uses exponents g_r - g_i with r >= i ("Sparse Delta
  Memory: layer and kernels", section "What the layer computes": the masked,
  exact chunk form), so every output must stay finite and match the oracle.
- NaN propagation.  Nothing is clipped: a NaN written into one value channel of
  one token reaches every later output of that channel and the final state, and
  nothing else (the rows of S evolve independently, one per value channel).  The
  chunk form multiplies masked zeros, so inside the NaN's own chunk the earlier
  tokens of that channel may turn NaN as well; every chunk before it, every other
  channel and every other stream must be bitwise what a clean call gives.
- Ill-conditioned solve.  Correlated keys (k_r . k_i ~ 0.99), runs of repeated
  keys and beta near 1 make I + tril(beta A, -1) far from the identity, where the
  inverse amplifies rounding ("Sparse Delta Memory: layer and kernels", section
  "Precision").  The bf16 path must still meet the 2e-2 bar, fp32 the 1e-5 bar.
- Caller streams.  Work enqueued on a stream other than torch's current one must
  keep the scratch the binding allocated alive until that stream has used it.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunked_amd import (chunk_bwd, chunk_fwd, chunk_fwd_segmented,
                                                   chunk_fwd_varlen, decode_step)
from linear_attention_sequence_chunked_amd.workloads import make_inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
DEV = torch.device("cuda:0")
GRADS = ("dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state")


def dev(inp):
    return {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}


def finite(*ts):
    return all(bool(torch.isfinite(t).all()) for t in ts if t is not None)


def masked_exponent_overflows(alpha, chunk):
    """True when, in some chunk, 2^(g_i - g_r) for a masked pair i > r would be
    above float32's range (exponent > 128): exponentiating before masking would
    give inf there."""
    la = -np.log2(alpha.double().numpy())      # [B, T, H], >= 0
    T = la.shape[1]
    worst = 0.0
    for t0 in range(0, T, chunk):
        # largest g_i - g_r over i > r in the chunk: the decay of its tokens after the first
        worst = max(worst, float(la[:, t0 + 1:t0 + chunk].sum(1).max(initial=0.0)))
    return worst > 128.0


def fwd_parity(inp, chunk, tol, label):
    print("case %s shape=%s dtype=%s chunk=%d" % (label, tuple(inp["q"].shape), inp["q"].dtype,
                                                   chunk), flush=True)
    g = dev(inp)
    o, sf = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"], chunk=chunk)
    torch.cuda.synchronize()
    assert finite(o, sf), label
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity(label, {"o": (o, ro), "final_state": (sf, rs)}, tol)


def bwd_parity(inp, chunk, tol, label, d_sf=None):
    print("case %s shape=%s dtype=%s chunk=%d" % (label, tuple(inp["q"].shape), inp["q"].dtype,
                                                   chunk), flush=True)
    g = dev(inp)
    got = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                    d_sf.to(DEV) if d_sf is not None else None, chunk=chunk)
    torch.cuda.synchronize()
    assert finite(*got), label
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["d_o"],
                     inp["initial_state"], d_sf)
    assert_parity(label, {n: (x, ref[n]) for n, x in zip(GRADS, got)}, tol)


# ------------------------------------------------------------------ strong decay

def gate_for(chunk):
    # alpha in (0.005, 0.2) overflows a masked exponent in 64-token chunks; shorter
    # chunks need alpha in (2^-16, 2^-4)
    return "strong" if chunk == 64 else "extreme"


STRONG_FWD = [
    # (B, T, H, K, V, chunk, dtype)
    (2, 300, 2, 128, 128, 64, torch.bfloat16),
    (1, 200, 3, 64, 32, 32, torch.bfloat16),
    (1, 150, 2, 32, 64, 16, torch.bfloat16),
    (2, 300, 2, 128, 128, 64, torch.float32),
    (1, 150, 2, 64, 16, 32, torch.float32),
]


@pytest.mark.parametrize("case", STRONG_FWD, ids=lambda c: "B%dT%dH%dK%dV%dC%d%s" % (
    c[:6] + ("f32" if c[6] == torch.float32 else "bf16",)))
def test_strong_decay_forward(case):
    B, T, H, K, V, C, dt = case
    inp = make_inputs(B, T, H, K, V, dtype=dt, seed=1200 + T + K, gate=gate_for(C), s0_std=0.1)
    assert masked_exponent_overflows(inp["alpha"], C)
    fwd_parity(inp, C, TOL[dt], "strong decay forward")


STRONG_BWD = [
    (2, 200, 2, 128, 128, 64, torch.bfloat16),   # matrix-core backward
    (1, 130, 2, 64, 32, 64, torch.bfloat16),
    (1, 100, 2, 16, 32, 32, torch.bfloat16),     # K = 16: float32 path with bf16 tensors
    (1, 150, 2, 64, 64, 32, torch.float32),      # float32 path
    (2, 70, 1, 128, 16, 64, torch.float32),
]


@pytest.mark.parametrize("case", STRONG_BWD, ids=lambda c: "B%dT%dH%dK%dV%dC%d%s" % (
    c[:6] + ("f32" if c[6] == torch.float32 else "bf16",)))
def test_strong_decay_backward(case):
    B, T, H, K, V, C, dt = case
    # the matrix-core backward always takes 64-token chunks; the float32 path
    # takes min(chunk, 32)
    bc = 64 if (dt == torch.bfloat16 and K >= 32 and V >= 32) else min(C, 32)
    inp = make_inputs(B, T, H, K, V, dtype=dt, seed=1300 + T + K, gate=gate_for(bc), s0_std=0.1,
                      with_do=True)
    assert masked_exponent_overflows(inp["alpha"], bc)
    d_sf = torch.randn(B, H, V, K, generator=torch.Generator().manual_seed(1301)) * 0.1
    bwd_parity(inp, C, TOL[dt], "strong decay backward", d_sf)


@pytest.mark.parametrize("dt,C", [(torch.bfloat16, 64), (torch.float32, 32)])
def test_strong_decay_segmented(dt, C):
    inp = make_inputs(1, 700, 2, 128, 64, dtype=dt, seed=1400, gate=gate_for(C), s0_std=0.1)
    assert masked_exponent_overflows(inp["alpha"], C)
    print("case strong decay segmented %s" % dt, flush=True)
    g = dev(inp)
    o, sf = chunk_fwd_segmented(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"],
                                chunk=C, segments=5)
    torch.cuda.synchronize()
    assert finite(o, sf)
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("strong decay segmented", {"o": (o, ro), "final_state": (sf, rs)}, TOL[dt])


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_strong_decay_varlen(dt):
    lengths = [130, 1, 64, 257]
    print("case strong decay varlen %s %s" % (dt, lengths), flush=True)
    C = 64 if dt == torch.bfloat16 else 32
    parts = [make_inputs(1, L, 2, 64, 64, dtype=dt, seed=1500 + i, gate=gate_for(C), s0_std=0.1)
             for i, L in enumerate(lengths)]
    cat = {n: torch.cat([p[n] for p in parts], 1) for n in ("q", "k", "v", "alpha", "beta")}
    s0 = torch.cat([p["initial_state"] for p in parts], 0)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    g = dev(cat)
    o, sf = chunk_fwd_varlen(g["q"], g["k"], g["v"], g["alpha"], g["beta"], cu.to(DEV), s0.to(DEV),
                             chunk=C)
    torch.cuda.synchronize()
    assert finite(o, sf)
    for i, p in enumerate(parts):
        ro, rs = oracle.fwd(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["initial_state"])
        a, b = int(cu[i]), int(cu[i + 1])
        assert_parity("strong decay varlen seq %d" % i,
                      {"o": (o[:, a:b], ro), "final_state": (sf[i:i + 1], rs)}, TOL[dt])


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_strong_decay_decode(dt):
    inp = make_inputs(3, 6, 4, 128, 64, dtype=dt, seed=1600, gate="extreme", s0_std=0.3)
    print("case strong decay decode %s" % dt, flush=True)
    state = inp["initial_state"].to(DEV).clone()
    g = dev(inp)
    outs = [decode_step(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(), g["v"][:, t].contiguous(),
                        g["alpha"][:, t].contiguous(), g["beta"][:, t].contiguous(), state)
            for t in range(inp["q"].shape[1])]
    torch.cuda.synchronize()
    o = torch.stack(outs, 1)
    assert finite(o, state)
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("strong decay decode o", {"o": (o, ro)}, TOL[dt])
    assert_parity("strong decay decode state", {"final_state": (state, rs)}, 1e-5)


# ------------------------------------------------------------- NaN propagation

@pytest.mark.parametrize("dt,C,entry", [(torch.bfloat16, 64, "plain"), (torch.float32, 32, "plain"),
                                        (torch.bfloat16, 64, "segmented"),
                                        (torch.float32, 16, "segmented")])
def test_nan_in_one_value_propagates_forward_only(dt, C, entry):
    B, T, H, K, V = 2, 300, 3, 64, 64
    b0, t0, h0, j0 = 1, 150, 2, 37
    inp = make_inputs(B, T, H, K, V, dtype=dt, seed=1700, s0_std=0.1)
    print("case NaN %s %s chunk=%d at (b=%d, t=%d, h=%d, j=%d)" % (entry, dt, C, b0, t0, h0, j0),
          flush=True)
    g = dev(inp)
    bad = g["v"].clone()
    bad[b0, t0, h0, j0] = float("nan")

    def call(v):
        if entry == "plain":
            return chunk_fwd(g["q"], g["k"], v, g["alpha"], g["beta"], g["initial_state"], chunk=C)
        return chunk_fwd_segmented(g["q"], g["k"], v, g["alpha"], g["beta"], g["initial_state"],
                                   chunk=C, segments=3)

    o_ref, s_ref = call(g["v"])
    o_bad, s_bad = call(bad)
    torch.cuda.synchronize()
    assert finite(o_ref, s_ref)
    # later outputs of the channel and its final-state row carry the NaN
    assert bool(torch.isnan(o_bad[b0, t0:, h0, j0]).all())
    assert bool(torch.isnan(s_bad[b0, h0, j0]).all())
    # everything else is bitwise the clean result
    keep = torch.ones_like(o_ref, dtype=torch.bool)
    keep[b0, (t0 // C) * C:, h0, j0] = False
    assert torch.equal(o_bad[keep], o_ref[keep])
    keep_s = torch.ones_like(s_ref, dtype=torch.bool)
    keep_s[b0, h0, j0] = False
    assert torch.equal(s_bad[keep_s], s_ref[keep_s])


# ----------------------------------------------------------- ill-conditioned

ILL = [
    # (keys, beta range, dtype, chunk)
    ("correlated", (0.9, 1.0), torch.bfloat16, 64),
    ("repeated", (0.9, 1.0), torch.bfloat16, 64),
    ("repeated", (1.0, 1.0), torch.bfloat16, 64),
    ("correlated", (0.9, 1.0), torch.bfloat16, 32),
    ("correlated", (0.9, 1.0), torch.float32, 32),
    ("repeated", (1.0, 1.0), torch.float32, 64),
]


@pytest.mark.parametrize("case", ILL, ids=lambda c: "%s-b%g-%g-%s-C%d" % (
    c[0], c[1][0], c[1][1], "f32" if c[2] == torch.float32 else "bf16", c[3]))
@pytest.mark.parametrize("gate", ["decay", "sigmoid"])
def test_ill_conditioned_solve_forward(case, gate):
    keys, br, dt, C = case
    inp = make_inputs(2, 400, 3, 128, 128, dtype=dt, seed=1800 + C, gate=gate, s0_std=0.05,
                      keys=keys, beta_range=br)
    fwd_parity(inp, C, TOL[dt], "ill-conditioned forward %s %s" % (keys, br))


@pytest.mark.parametrize("case", ILL[:3] + ILL[4:5], ids=lambda c: "%s-b%g-%g-%s" % (
    c[0], c[1][0], c[1][1], "f32" if c[2] == torch.float32 else "bf16"))
def test_ill_conditioned_solve_backward(case):
    keys, br, dt, C = case
    inp = make_inputs(2, 260, 2, 128, 128 if dt == torch.bfloat16 else 64, dtype=dt, seed=1900,
                      s0_std=0.05, keys=keys, beta_range=br, with_do=True)
    bwd_parity(inp, C, TOL[dt], "ill-conditioned backward %s %s" % (keys, br))


def test_forward_train_shape_correlated_keys_sampled():
    # the training shape's sizes (B8 T4096 H6 d128) with correlated keys and
    # beta in [0.9, 1], checked on a sample of four streams
    B, T, H = 8, 4096, 6
    inp = make_inputs(B, T, H, 128, 128, dtype=torch.bfloat16, seed=1950, keys="correlated",
                      beta_range=(0.9, 1.0))
    print("case ill-conditioned training shape", flush=True)
    g = dev(inp)
    o, sf = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], None, chunk=64)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 5), (7, 2), (5, 1)):
        sl = {n: inp[n][b:b + 1, :, h:h + 1].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        ro, rs = oracle.fwd(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["beta"], None)
        assert_parity("stream (%d, %d)" % (b, h),
                      {"o": (o[b:b + 1, :, h:h + 1], ro), "final_state": (sf[b:b + 1, h:h + 1], rs)},
                      2e-2)


# ------------------------------------------------------------- caller streams

def _busy(stream):
    # queue a few milliseconds of work on `stream` so that what follows on it
    # starts late, after the host has returned and reused freed memory
    with torch.cuda.stream(stream):
        x = torch.randn(2048, 2048, device=DEV)
        for _ in range(20):
            x = x @ x
            x = x / x.norm()


def _churn(nbytes):
    # allocate and overwrite memory on torch's current stream, as a caller would
    for n in (nbytes, nbytes // 2, nbytes):
        t = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
        t.fill_(0xA5)
        del t


def test_backward_on_an_explicit_stream_keeps_its_workspace():
    inp = make_inputs(2, 300, 3, 128, 128, dtype=torch.bfloat16, seed=2100, s0_std=0.05, with_do=True)
    g = dev(inp)
    args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"])
    ref = chunk_bwd(*args, chunk=64)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for trial in range(3):
        _busy(s)
        got = chunk_bwd(*args, chunk=64, stream=s)
        _churn(64 << 20)
        s.synchronize()
        torch.cuda.synchronize()
        for n, x, y in zip(GRADS, ref, got):
            assert torch.equal(x, y), (trial, n)


def test_segmented_on_an_explicit_stream_keeps_its_workspace():
    inp = make_inputs(1, 2000, 2, 128, 128, dtype=torch.bfloat16, seed=2200, s0_std=0.05)
    g = dev(inp)
    args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"])
    ref = chunk_fwd_segmented(*args, chunk=64, segments=8)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for trial in range(3):
        _busy(s)
        got = chunk_fwd_segmented(*args, chunk=64, segments=8, stream=s)
        _churn(16 << 20)
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1]), trial
