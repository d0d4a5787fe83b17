"""The allocation-free segmented forward (gdn_chunk_fwd_segmented_noalloc)
against the segmented forward with a caller workspace, through the C ABI.

Two calls in a row share the library's static scratch, the second with a
smaller input: each must equal the workspace call (bitwise for bfloat16: same
kernels, same arithmetic; within 1e-5 relative L2 for float32, where the
workspace call runs on the fp32 matrix cores with pooled factors and the
allocation-free call on the scalar fp32 kernel) and meet the oracle's bar (1e-5
float32, 2e-2 bfloat16 relative L2, whole tensor and every local block).  The result of the first call is checked
after the second has run, so a second call that wrote into the first call's
outputs, or read stale scratch, would show.
"""
import pytest
import torch

import oracle
from linear_attention_sequence_chunked_amd import chunk_fwd_segmented, chunk_fwd_segmented_noalloc
from linear_attention_sequence_chunked_amd.gdn import SEGMENTED_NOALLOC_MAX_BYTES, segmented_workspace_size
from linear_attention_sequence_chunked_amd.workloads import make_inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def dev(inp):
    return {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}


def args(g):
    return (g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"])


@pytest.mark.parametrize("dt,C", [(torch.bfloat16, 64), (torch.float32, 32)])
def test_noalloc_matches_workspace_call_twice_in_a_row(dt, C):
    big = make_inputs(1, 3000, 4, 128, 128, dtype=dt, seed=2300, s0_std=0.05)
    small = make_inputs(2, 700, 2, 64, 32, dtype=dt, seed=2301, s0_std=0.1)
    print("case noalloc %s: B1 T3000 H4 d128 P8, then B2 T700 H2 K64 V32 P5" % dt, flush=True)
    assert segmented_workspace_size(1, 3000, 4, 128, 128, C, 8) <= SEGMENTED_NOALLOC_MAX_BYTES
    gb, gs = dev(big), dev(small)
    ref_b = chunk_fwd_segmented(*args(gb), chunk=C, segments=8)
    ref_s = chunk_fwd_segmented(*args(gs), chunk=C, segments=5)
    torch.cuda.synchronize()
    got_b = chunk_fwd_segmented_noalloc(*args(gb), chunk=C, segments=8)
    got_s = chunk_fwd_segmented_noalloc(*args(gs), chunk=C, segments=5)
    torch.cuda.synchronize()
    for name, got, ref in (("first", got_b, ref_b), ("second", got_s, ref_s)):
        if dt == torch.bfloat16:
            assert torch.equal(got[0], ref[0]), name
            assert torch.equal(got[1], ref[1]), name
        else:
            for x, y in zip(got, ref):
                err = float((x.double() - y.double()).norm() / y.double().norm())
                assert err <= 1e-5, (name, err)
    for inp, got in ((big, got_b), (small, got_s)):
        ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                            inp["initial_state"])
        assert_parity("noalloc", {"o": (got[0], ro), "final_state": (got[1], rs)}, TOL[dt])


def test_noalloc_with_caller_outputs_and_in_place_state():
    # outputs passed in and the state advanced in place: nothing allocated per call
    inp = make_inputs(1, 2000, 2, 128, 128, dtype=torch.bfloat16, seed=2310, s0_std=0.05)
    g = dev(inp)
    ref_o, ref_s = chunk_fwd_segmented(*args(g), chunk=64, segments=6)
    out = torch.empty_like(ref_o)
    state = g["initial_state"].clone()
    torch.cuda.synchronize()
    o, s = chunk_fwd_segmented_noalloc(g["q"], g["k"], g["v"], g["alpha"], g["beta"], state, chunk=64,
                                       segments=6, out=out, final_state=state)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and s.data_ptr() == state.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(state, ref_s)


def test_noalloc_refuses_more_than_its_scratch():
    inp = make_inputs(1, 64, 1, 16, 16, dtype=torch.bfloat16, seed=2320)
    g = dev(inp)
    # 64 segments of one chunk each need little; a long 16-head call with 64
    # segments needs far more than 64 MiB: refused on the host, nothing launched
    q = torch.empty(1, 32768, 16, 128, dtype=torch.bfloat16, device=DEV)
    a = torch.full((1, 32768, 16), 0.9, device=DEV)
    assert segmented_workspace_size(1, 32768, 16, 128, 128, 64, 64) > SEGMENTED_NOALLOC_MAX_BYTES
    with pytest.raises(MemoryError):
        chunk_fwd_segmented_noalloc(q, q, q, a, a, None, chunk=64, segments=64)
    o, s = chunk_fwd_segmented_noalloc(*args(g), chunk=16, segments=4)
    torch.cuda.synchronize()
    ref = chunk_fwd_segmented(*args(g), chunk=16, segments=4)
    assert torch.equal(o, ref[0]) and torch.equal(s, ref[1])


def test_noalloc_single_segment_float32_allocates_nothing_and_matches():
    # one segment is the plain call; without allocation float32 takes the scalar
    # kernel (the plain call's matrix-core path draws pooled factors)
    inp = make_inputs(2, 500, 3, 64, 64, dtype=torch.float32, seed=2330, s0_std=0.1)
    print("case noalloc float32 single segment", flush=True)
    g = dev(inp)
    o, s = chunk_fwd_segmented_noalloc(*args(g), chunk=32, segments=1)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    assert_parity("noalloc single segment", {"o": (o, ro), "final_state": (s, rs)}, 1e-5)
