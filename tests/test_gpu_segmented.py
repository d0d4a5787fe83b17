"""Segment-parallel forward (gdn_chunk_fwd_segmented) through the C ABI.

Every sequence is cut into P segments joined by their affine state maps; the
result must match the fp64 oracle like the plain forward (1e-5 float32 / 2e-2
bfloat16 relative L2 on o and the final state), including ragged and empty
segments, P = 1, and the state advanced in place.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunked_amd import chunk_fwd, chunk_fwd_segmented
from linear_attention_sequence_chunked_amd.workloads import WORKLOADS, make_inputs, workload_inputs

from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
DEV = torch.device("cuda:0")


def rel_l2(x, ref):
    x = x.detach().double().cpu().numpy()
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


CASES = [
    # (B, T, H, K, V, chunk, dtype, s0_std, segments)
    (1, 1000, 2, 128, 128, 64, torch.bfloat16, 0.05, 4),
    (2, 333, 3, 64, 32, 32, torch.float32, 0.2, 3),
    (1, 100, 2, 128, 64, 64, torch.bfloat16, 0.1, 8),     # empty trailing segments
    (3, 257, 1, 32, 32, 16, torch.bfloat16, None, 5),
    (1, 777, 2, 16, 64, 16, torch.float32, 0.3, 7),
    (2, 500, 2, 128, 128, 64, torch.float32, 0.05, 1),    # the plain path
    (2, 300, 2, 64, 16, 32, torch.float32, 0.2, 2),       # one transition
    # bf16, 64-token chunks, K and V in {64, 128}: both states-only passes in one
    # launch with 64 value rows per workgroup
    (2, 700, 3, 64, 128, 64, torch.bfloat16, 0.1, 5),
    (1, 500, 2, 64, 64, 64, torch.bfloat16, None, 3),
    (3, 450, 2, 128, 64, 64, torch.bfloat16, 0.05, 2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dK%dV%dC%dP%d%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[8], "f32" if c[6] == torch.float32 else "bf16"))
def test_segmented_matches_oracle(case):
    B, T, H, K, V, C, dt, s0, P = case
    inp = make_inputs(B, T, H, K, V, dtype=dt, seed=600 + T, gate="decay", s0_std=s0)
    print("case segmented %s" % (case,), flush=True)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    o, sf = chunk_fwd_segmented(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"],
                                chunk=C, segments=P)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("segmented", {"o": (o, ro), "final_state": (sf, rs)}, TOL[dt])


def test_segmented_state_in_place_and_close_to_plain():
    inp = make_inputs(1, 600, 4, 128, 128, dtype=torch.bfloat16, seed=611, s0_std=0.05)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    o1, s1 = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"], chunk=64)
    state = g["initial_state"].clone()
    o2, s2 = chunk_fwd_segmented(g["q"], g["k"], g["v"], g["alpha"], g["beta"], state, chunk=64,
                                 segments=3, final_state=state)
    torch.cuda.synchronize()
    assert s2.data_ptr() == state.data_ptr()
    assert rel_l2(o2, o1.double().cpu().numpy()) <= 1e-2
    assert rel_l2(s2, s1.double().cpu().numpy()) <= 1e-2


@pytest.mark.parametrize("P", [4, 8, 2])
def test_long_context_workload_segmented(P):
    # the full long-context workload; its two states-only passes run in one launch of
    # 16 P (V/64 + K/64) workgroups: 256 at P = 4, 512 (more than the CUs) at P = 8
    w = WORKLOADS["long_bf16"]
    inp = workload_inputs(w)
    print("case long-context segmented P=%d" % P, flush=True)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    o, sf = chunk_fwd_segmented(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"],
                                chunk=w.chunk, segments=P)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("long segmented", {"o": (o, ro), "final_state": (sf, rs)}, 2e-2)


@pytest.mark.parametrize("K,P", [(64, 6), (128, 9), (32, 2)])
def test_segmented_weak_decay_carries_state_across_segments(K, P):
    # alpha in (0.995, 1) and small beta: the state carries across hundreds of
    # tokens, so every segment's output depends on the transition A_s of the
    # segments before it
    inp = make_inputs(2, 900, 2, K, 64, dtype=torch.float32, seed=620 + K, s0_std=0.3)
    g = torch.Generator().manual_seed(621)
    inp["alpha"] = 1.0 - 0.005 * torch.rand(inp["alpha"].shape, generator=g)
    inp["beta"] = 0.1 * torch.rand(inp["beta"].shape, generator=g)
    gd = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    o, sf = chunk_fwd_segmented(gd["q"], gd["k"], gd["v"], gd["alpha"], gd["beta"],
                                gd["initial_state"], chunk=32, segments=P)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("weak decay", {"o": (o, ro), "final_state": (sf, rs)}, 1e-5)


def test_segment_count_from_the_hint():
    # segments=None takes gdn_chunk_fwd_segments_hint for the device; on a
    # few-stream sequence it splits, and the result still matches the oracle
    inp = make_inputs(1, 4096, 2, 128, 128, dtype=torch.bfloat16, seed=630, s0_std=0.05)
    from linear_attention_sequence_chunked_amd import segments_hint
    P = segments_hint(1, 4096, 2, 128, 128, 64)
    print("hint for B1 T4096 H2: %d segments" % P, flush=True)
    assert P > 1
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    o, sf = chunk_fwd_segmented(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"],
                                chunk=64)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("hinted", {"o": (o, ro), "final_state": (sf, rs)}, TOL[torch.bfloat16])


@pytest.mark.parametrize("K,V,P", [(64, 64, 6), (128, 128, 9), (128, 64, 4)])
def test_segmented_weak_decay_bf16_merged_passes(K, V, P):
    # the bf16 states-only passes (N and A in one launch): with alpha in (0.995, 1)
    # every segment's output depends on the transitions of the segments before it
    inp = make_inputs(2, 1100, 2, K, V, dtype=torch.bfloat16, seed=640 + K + V, s0_std=0.3)
    g = torch.Generator().manual_seed(641)
    inp["alpha"] = 1.0 - 0.005 * torch.rand(inp["alpha"].shape, generator=g)
    inp["beta"] = 0.1 * torch.rand(inp["beta"].shape, generator=g)
    print("case weak decay bf16 K%d V%d P%d" % (K, V, P), flush=True)
    gd = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    o, sf = chunk_fwd_segmented(gd["q"], gd["k"], gd["v"], gd["alpha"], gd["beta"],
                                gd["initial_state"], chunk=64, segments=P)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("weak decay bf16", {"o": (o, ro), "final_state": (sf, rs)}, TOL[torch.bfloat16])
