"""Parity of the HIP decode step (through the C ABI) with the fp64 token oracle.

One decode call is one token of the recurrence with the state advanced in place,
so k calls must equal the oracle's forward over those k tokens, and a decode
continuing a chunked prefill must equal the oracle over prefill + decode tokens.
o is compared at 1e-5 (float32) / 2e-2 (bfloat16) relative L2; the state is
float32 arithmetic for both dtypes and is compared at 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunked_amd import chunk_fwd, decode_step
from linear_attention_sequence_chunked_amd.workloads import WORKLOADS, make_inputs, workload_inputs

from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
DEV = torch.device("cuda:0")


def rel_l2(x, ref):
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x)
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def run_decode(inp, state):
    """Feed every token of inp through decode_step; returns o [B,T,H,V] (device)."""
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    T = g["q"].shape[1]
    outs = []
    for t in range(T):
        outs.append(decode_step(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(),
                                g["v"][:, t].contiguous(), g["alpha"][:, t].contiguous(),
                                g["beta"][:, t].contiguous(), state))
    torch.cuda.synchronize()
    return torch.stack(outs, 1)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K,V", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
def test_decode_steps_match_oracle(dt, K, V):
    inp = make_inputs(2, 7, 3, K, V, dtype=dt, seed=40 + K + V, gate="sigmoid", s0_std=0.2)
    print("case decode K=%d V=%d %s" % (K, V, dt), flush=True)
    state = inp["initial_state"].to(DEV).clone()
    o = run_decode(inp, state)
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("decode o", {"o": (o, ro)}, TOL[dt])
    assert_parity("decode state", {"final_state": (state, rs)}, 1e-5)


def test_decode_continues_a_prefill():
    # chunked prefill of 300 tokens, then 20 decode steps == one 320-token stream
    inp = make_inputs(2, 320, 4, 128, 128, dtype=torch.bfloat16, seed=44, s0_std=0.05)
    pre = {n: (t[:, :300].contiguous() if t is not None and n != "initial_state" else t)
           for n, t in inp.items()}
    dec = {n: (t[:, 300:].contiguous() if t is not None and n != "initial_state" else t)
           for n, t in inp.items()}
    g = {n: (t.to(DEV) if t is not None else None) for n, t in pre.items()}
    o1, state = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"], chunk=64)
    o2 = run_decode(dec, state)
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("prefill+decode", {"o": (torch.cat([o1, o2], 1), ro), "final_state": (state, rs)}, 2e-2)
    assert rel_l2(o2, ro[:, 300:]) <= 2e-2


def test_decode_workload_one_step():
    w = WORKLOADS["decode_bf16"]
    inp = workload_inputs(w)
    state = inp["initial_state"].to(DEV).clone()
    o = run_decode(inp, state)
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("decode workload o", {"o": (o, ro)}, 2e-2)
    assert_parity("decode workload state", {"final_state": (state, rs)}, 1e-5)


def test_decode_identity_gates_keep_state_and_read_it():
    # alpha = 1, beta = 0: the state is unchanged (bitwise) and o = S q
    inp = make_inputs(1, 1, 2, 64, 64, dtype=torch.float32, seed=45, s0_std=0.3)
    inp["alpha"] = torch.ones_like(inp["alpha"])
    inp["beta"] = torch.zeros_like(inp["beta"])
    s0 = inp["initial_state"].to(DEV)
    state = s0.clone()
    o = run_decode(inp, state)
    assert torch.equal(state, s0)
    ref = torch.einsum("bhvk,bhk->bhv", inp["initial_state"].double(), inp["q"][:, 0].double())
    assert rel_l2(o[:, 0], ref.numpy()) <= 1e-6
