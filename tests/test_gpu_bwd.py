"""Parity of the HIP backward (through the C ABI) with the oracle's fp64 reverse mode.

Loss L = <o, d_o> + <final_state, d_final_state>.  Every gradient (dq, dk, dv,
dalpha, dbeta, d_initial_state) is compared by relative L2 in fp64, over the
whole tensor and over every local block (each (batch, head, 64-token block) of
dq, dk, dv; each (batch, head) of the gate and state gradients; tests/parity.py):
<= 1e-5 for float32 inputs, <= 2e-2 for bfloat16 inputs (the oracle reads the
same rounded values).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunked_amd import bwd_workspace_size, chunk_bwd
from linear_attention_sequence_chunked_amd.workloads import WORKLOADS, make_inputs, workload_inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
DEV = torch.device("cuda:0")
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state")


def rel_l2(x, ref):
    x = x.detach().double().cpu().numpy()
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def gpu_bwd(inp, chunk, d_sf=None):
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    out = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                    d_sf.to(DEV) if d_sf is not None else None, chunk=chunk)
    torch.cuda.synchronize()
    return dict(zip(NAMES, out))


def check(inp, chunk, tol, label, d_sf=None):
    print("case %s chunk=%d shape=%s dtype=%s" % (label, chunk, tuple(inp["q"].shape),
                                                   inp["q"].dtype), flush=True)
    got = gpu_bwd(inp, chunk, d_sf)
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["d_o"],
                     inp["initial_state"], d_sf)
    assert_parity(label, {n: (got[n], ref[n]) for n in NAMES}, tol)
    return got


def test_tiny_fp32_with_final_state_gradient():
    w = WORKLOADS["tiny_fp32"]
    inp = workload_inputs(w)
    inp["d_o"] = torch.randn(inp["v"].shape, generator=torch.Generator().manual_seed(11))
    d_sf = torch.randn(1, 2, 16, 16, generator=torch.Generator().manual_seed(12))
    check(inp, w.chunk, TOL[torch.float32], "tiny", d_sf)


BWD_SWEEP = [
    # (B, T, H, K, V, chunk, dtype, s0_std)
    (1, 1, 1, 16, 16, 16, torch.float32, 0.5),
    (2, 17, 3, 32, 16, 16, torch.float32, None),
    (1, 130, 2, 64, 32, 32, torch.float32, 0.1),
    (1, 200, 2, 128, 128, 64, torch.float32, 0.05),
    (2, 50, 2, 16, 64, 32, torch.float32, 0.3),
    # 16-token chunks through the one-launch walks; more workgroups than CUs there
    (2, 70, 3, 64, 64, 16, torch.float32, 0.2),
    (8, 96, 6, 128, 128, 32, torch.float32, None),
    (1, 1, 2, 128, 128, 64, torch.bfloat16, 0.1),
    (1, 63, 2, 128, 128, 64, torch.bfloat16, None),
    (2, 65, 3, 128, 128, 64, torch.bfloat16, 0.02),
    (1, 300, 2, 128, 64, 64, torch.bfloat16, 0.05),
    (1, 257, 4, 64, 64, 32, torch.bfloat16, 0.05),
    (3, 100, 1, 32, 32, 16, torch.bfloat16, 0.05),
]


@pytest.mark.parametrize("case", BWD_SWEEP, ids=lambda c: "B%dT%dH%dK%dV%dC%d%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "f32" if c[6] == torch.float32 else "bf16"))
@pytest.mark.parametrize("gate", ["decay", "sigmoid"])
def test_bwd_shape_sweep(case, gate):
    B, T, H, K, V, C, dt, s0 = case
    inp = make_inputs(B, T, H, K, V, dtype=dt, seed=300 + T + K, gate=gate, s0_std=s0, with_do=True)
    d_sf = torch.randn(B, H, V, K, generator=torch.Generator().manual_seed(T)) * 0.1
    check(inp, C, TOL[dt], "sweep", d_sf)


# bf16 inputs with K, V >= 32 take the MFMA backward (64-token chunks): every
# compiled (K, V) pair, ragged tails, several chunks
MFMA_SWEEP = [
    # (B, T, H, K, V, chunk)
    (2, 129, 2, 32, 32, 64),
    (1, 200, 3, 64, 128, 64),
    (1, 192, 2, 32, 128, 64),
    (1, 100, 2, 128, 32, 64),
    (2, 64, 1, 64, 32, 64),
    (1, 77, 2, 32, 64, 64),
    (1, 250, 2, 128, 128, 64),
]


@pytest.mark.parametrize("case", MFMA_SWEEP, ids=lambda c: "B%dT%dH%dK%dV%dC%d" % c)
@pytest.mark.parametrize("gate", ["decay", "sigmoid"])
def test_bwd_mfma_shapes(case, gate):
    B, T, H, K, V, C = case
    inp = make_inputs(B, T, H, K, V, dtype=torch.bfloat16, seed=700 + T + K + V, gate=gate,
                      s0_std=0.05, with_do=True)
    d_sf = torch.randn(B, H, V, K, generator=torch.Generator().manual_seed(T + 1)) * 0.1
    check(inp, C, TOL[torch.bfloat16], "mfma", d_sf)


def test_bwd_reproducible_and_workspace_reuse():
    inp = make_inputs(2, 150, 2, 64, 64, dtype=torch.bfloat16, seed=21, s0_std=0.05, with_do=True)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    ws = torch.empty(bwd_workspace_size(2, 150, 2, 64, 64, 64, dtype=torch.bfloat16), dtype=torch.uint8,
                     device=DEV)
    a = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                  chunk=64, workspace=ws)
    ws.fill_(0xFF)  # stale contents must not matter
    b = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                  chunk=64, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_zero_upstream_gives_zero_gradients():
    inp = make_inputs(1, 90, 2, 32, 32, dtype=torch.float32, seed=22, s0_std=0.1, with_do=True)
    inp["d_o"] = torch.zeros_like(inp["d_o"])
    got = gpu_bwd(inp, 32)
    for n in NAMES:
        assert torch.count_nonzero(got[n]).item() == 0, n


def test_bwd_mfma_zero_upstream_gives_zero_gradients():
    inp = make_inputs(2, 130, 2, 128, 64, dtype=torch.bfloat16, seed=23, s0_std=0.1, with_do=True)
    inp["d_o"] = torch.zeros_like(inp["d_o"])
    got = gpu_bwd(inp, 64)
    for n in NAMES:
        assert torch.count_nonzero(got[n]).item() == 0, n


def test_fwdbwd_workload_parity():
    # the forward+backward shape: B4 T2048 H6 K=V=128 bf16, d_final_state = 0
    w = WORKLOADS["fwdbwd_bf16"]
    check(workload_inputs(w), w.chunk, TOL[w.dtype], w.name)


def test_fwdbwd_f32_workload_parity():
    # the same shape with float32 q, k, v, d_o: 32-token chunks with the state
    # recompute, reverse walk and token gradients on the fp32 matrix cores
    w = WORKLOADS["fwdbwd_f32"]
    check(workload_inputs(w), w.chunk, TOL[w.dtype], w.name)


def test_bwd_mfma_more_chunks_than_compute_units():
    # the token-gradient kernel runs one workgroup per CU, each taking every
    # gridDim-th (chunk, head, batch): 2 x 133 chunks (a ragged last one) > 256
    # CUs, so some workgroups take two items and carry the prefetched operands of
    # the second
    inp = make_inputs(1, 64 * 132 + 17, 2, 64, 32, dtype=torch.bfloat16, seed=650, s0_std=0.05,
                      with_do=True)
    check(inp, 64, TOL[torch.bfloat16], "more chunks than CUs")


def test_bwd_mfma_walks_exceed_compute_units():
    # the two sequential walks share one launch of 2 x B*H*V/32 workgroups: here
    # 2 x 138 = 276 > 256 CUs (some wait for a free CU) and 138 is not a multiple
    # of 8 (neither half uses the XCD-aware numbering)
    inp = make_inputs(3, 150, 23, 64, 64, dtype=torch.bfloat16, seed=655, s0_std=0.05, with_do=True)
    check(inp, 64, TOL[torch.bfloat16], "walks launch larger than the GPU")


def test_bwd_writes_preallocated_results():
    inp = make_inputs(2, 150, 2, 64, 32, dtype=torch.bfloat16, seed=660, s0_std=0.05, with_do=True)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"])
    ref = chunk_bwd(*args, chunk=64)
    res = tuple(torch.full_like(x, float("nan")) for x in ref)
    got = chunk_bwd(*args, chunk=64, out=res)
    torch.cuda.synchronize()
    assert all(a is b for a, b in zip(got, res))
    for x, y in zip(ref, got):
        assert torch.equal(x, y)
    # d_initial_state skipped
    res2 = res[:5] + (None,)
    got2 = chunk_bwd(*args, chunk=64, out=res2)
    torch.cuda.synchronize()
    assert got2[5] is None
    for x, y in zip(ref[:5], got2[:5]):
        assert torch.equal(x, y)
    with pytest.raises(ValueError):
        chunk_bwd(*args, chunk=64, out=res[:5])
    with pytest.raises(ValueError):
        chunk_bwd(*args, chunk=64, out=(res[2],) + res[1:])   # a dq of the wrong shape


def test_bwd_mfma_on_a_side_stream_matches_default_stream():
    # the MFMA backward forks to a library stream and joins back; on a caller
    # stream other than the default the result must be the same bits
    inp = make_inputs(2, 200, 3, 128, 64, dtype=torch.bfloat16, seed=31, s0_std=0.05, with_do=True)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    ref = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"], chunk=64)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                        chunk=64)
    s.synchronize()
    for x, y in zip(ref, got):
        assert torch.equal(x, y)


def test_bwd_bf16_chunk_argument_keeps_the_mfma_path():
    # bf16 inputs with K, V >= 32 run the MFMA backward with 64-token chunks
    # whatever chunk is asked for, so every chunk gives the same bits
    inp = make_inputs(2, 150, 2, 64, 32, dtype=torch.bfloat16, seed=640, s0_std=0.05, with_do=True)
    outs = {C: gpu_bwd(inp, C) for C in (16, 32, 64)}
    for C in (16, 32):
        for n in NAMES:
            assert torch.equal(outs[C][n], outs[64][n]), (C, n)
    check(inp, 16, TOL[torch.bfloat16], "chunk16 on the MFMA path")
