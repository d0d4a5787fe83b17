"""Seeded sweep of random valid shapes through every entry point, against the
fp64 oracle.

The focused tests pick their shapes by hand; here each case draws batch, length,
heads, K, V (K != V allowed), chunk size, dtype, gate distribution and initial
state from a seeded generator, so that shapes nobody chose (ragged tails of every
length, single-token sequences, narrow heads with long chunks) meet the same bar:
relative L2 in fp64, over the whole tensor and over every local block (each
(batch, head, 64-token block) of a token tensor, each (batch, head) of a state or
gate gradient), <= 1e-5 for float32 inputs and <= 2e-2 for bfloat16 inputs.  Sizes stay small enough for the oracle to finish
each case in about a second.
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
WIDTHS = (16, 32, 64, 128)
GRAD_NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state")


def draw(seed, max_t=600, max_b=3, max_h=3):
    r = np.random.default_rng(seed)
    return dict(
        B=int(r.integers(1, max_b + 1)), T=int(r.integers(1, max_t + 1)), H=int(r.integers(1, max_h + 1)),
        K=int(r.choice(WIDTHS)), V=int(r.choice(WIDTHS)), chunk=int(r.choice((16, 32, 64))),
        dtype=(torch.float32, torch.bfloat16)[int(r.integers(2))],
        gate=("decay", "sigmoid")[int(r.integers(2))],
        s0=(None, 0.05, 0.3)[int(r.integers(3))])


def label(c):
    return "B%dT%dH%dK%dV%dC%d-%s-%s-s0%s" % (c["B"], c["T"], c["H"], c["K"], c["V"], c["chunk"],
                                              "f32" if c["dtype"] == torch.float32 else "bf16",
                                              c["gate"], c["s0"])


def inputs(c, seed, with_do=False):
    return make_inputs(c["B"], c["T"], c["H"], c["K"], c["V"], dtype=c["dtype"], seed=seed,
                       gate=c["gate"], s0_std=c["s0"], with_do=with_do)


def dev(inp):
    return {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}


def assert_close(tensors, tol, c):
    # whole-tensor and worst-block relative L2 (tests/parity.py)
    assert_parity(label(c), tensors, tol)


@pytest.mark.parametrize("seed", range(1000, 1016))
def test_random_forward(seed):
    c = draw(seed)
    print("case random forward seed=%d %s" % (seed, label(c)), flush=True)
    inp = inputs(c, seed)
    g = dev(inp)
    o, sf = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"], chunk=c["chunk"])
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_close({"o": (o, ro), "final_state": (sf, rs)}, TOL[c["dtype"]], c)


@pytest.mark.parametrize("seed", range(2000, 2006))
def test_random_ragged_batch(seed):
    c = draw(seed, max_b=1)
    r = np.random.default_rng(seed + 1)
    n = int(r.integers(1, 10))
    lengths = [int(x) for x in r.integers(0, 300, n)]
    print("case random varlen seed=%d %s lengths=%s" % (seed, label(c), lengths), flush=True)
    parts = [inputs(dict(c, B=1, T=max(L, 1)), seed + 10 + i) for i, L in enumerate(lengths)]
    for p, L in zip(parts, lengths):
        for nm in ("q", "k", "v", "alpha", "beta"):
            p[nm] = p[nm][:, :L].contiguous()
        if p["initial_state"] is None:
            p["initial_state"] = torch.zeros(1, c["H"], c["V"], c["K"])
    cat = {nm: torch.cat([p[nm] for p in parts], 1) for nm in ("q", "k", "v", "alpha", "beta")}
    s0 = torch.cat([p["initial_state"] for p in parts], 0)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    if int(cu[-1]) == 0:
        pytest.skip("all sequences empty")
    g = dev(cat)
    o, sf = chunk_fwd_varlen(g["q"], g["k"], g["v"], g["alpha"], g["beta"], cu.to(DEV), s0.to(DEV),
                             chunk=c["chunk"])
    torch.cuda.synchronize()
    for i, (p, L) in enumerate(zip(parts, lengths)):
        if L == 0:
            assert torch.equal(sf[i].cpu(), p["initial_state"][0])
            continue
        ro, rs = oracle.fwd(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["initial_state"])
        a, b = int(cu[i]), int(cu[i + 1])
        print("  sequence %d (%d tokens)" % (i, L), flush=True)
        assert_close({"o": (o[:, a:b], ro), "final_state": (sf[i:i + 1], rs)}, TOL[c["dtype"]], c)


@pytest.mark.parametrize("seed", range(3000, 3006))
def test_random_segmented(seed):
    c = draw(seed, max_t=900)
    P = int(np.random.default_rng(seed + 1).integers(1, min(c["T"], 12) + 1))
    print("case random segmented seed=%d %s segments=%d" % (seed, label(c), P), flush=True)
    inp = inputs(c, seed)
    g = dev(inp)
    o, sf = chunk_fwd_segmented(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"],
                                chunk=c["chunk"], segments=P)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_close({"o": (o, ro), "final_state": (sf, rs)}, TOL[c["dtype"]], c)


@pytest.mark.parametrize("seed", range(4000, 4008))
def test_random_backward(seed):
    c = draw(seed, max_t=400)
    print("case random backward seed=%d %s" % (seed, label(c)), flush=True)
    inp = inputs(c, seed, with_do=True)
    d_sf = torch.randn(c["B"], c["H"], c["V"], c["K"], generator=torch.Generator().manual_seed(seed)) * 0.1
    g = dev(inp)
    got = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                    d_sf.to(DEV), chunk=c["chunk"])
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["d_o"],
                     inp["initial_state"], d_sf)
    assert_close({n: (x, ref[n]) for n, x in zip(GRAD_NAMES, got)}, TOL[c["dtype"]], c)


@pytest.mark.parametrize("seed", range(5000, 5004))
def test_random_decode_steps(seed):
    c = draw(seed, max_t=8, max_b=6, max_h=4)
    print("case random decode seed=%d %s steps=%d" % (seed, label(c), c["T"]), flush=True)
    inp = inputs(dict(c, s0=0.3), seed)
    state = inp["initial_state"].to(DEV).clone()
    outs = []
    for t in range(c["T"]):
        o = decode_step(inp["q"][:, t].contiguous().to(DEV), inp["k"][:, t].contiguous().to(DEV),
                        inp["v"][:, t].contiguous().to(DEV), inp["alpha"][:, t].contiguous().to(DEV),
                        inp["beta"][:, t].contiguous().to(DEV), state)
        outs.append(o)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    o = torch.stack(outs, 1)
    assert_close({"o": (o, ro), "final_state": (state, rs)}, TOL[c["dtype"]], c)


@pytest.mark.parametrize("seed", range(4100, 4106))
def test_random_backward_mfma_path(seed):
    # bf16 inputs with 64-token chunks and K, V >= 32: the matrix-core backward
    r = np.random.default_rng(seed)
    c = dict(draw(seed, max_t=400), dtype=torch.bfloat16, chunk=64,
             K=int(r.choice((32, 64, 128))), V=int(r.choice((32, 64, 128))))
    print("case random backward (matrix cores) seed=%d %s" % (seed, label(c)), flush=True)
    inp = inputs(c, seed, with_do=True)
    d_sf = torch.randn(c["B"], c["H"], c["V"], c["K"], generator=torch.Generator().manual_seed(seed)) * 0.1
    g = dev(inp)
    got = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                    d_sf.to(DEV), chunk=64)
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["d_o"],
                     inp["initial_state"], d_sf)
    assert_close({n: (x, ref[n]) for n, x in zip(GRAD_NAMES, got)}, TOL[torch.bfloat16], c)
