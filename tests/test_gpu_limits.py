"""Parity at the largest sizes the forward accepts.

gdn.h caps every token tensor at B*T*H*max(K,V) < 2^31 elements and the state
at B*H*V*K <= 2^31; these cases sit at those caps (4.3 GB per bf16 token tensor,
tens of GB of device memory per case) so that every element offset the kernels
form reaches its largest value: one sequence of 1,048,575 tokens (a ragged last
chunk of 63 tokens), 8,192 sequences of two chunks with a state tensor at its own
cap (a grid of half a million workgroups), and a packed batch of the first case's
length.  The inputs are drawn on the device; the oracle checks a sample of whole
streams, copied back exactly as the GPU read them, against the same bar as the
smaller tests (relative L2 <= 2e-2 for bf16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunked_amd import chunk_fwd, chunk_fwd_varlen
from linear_attention_sequence_chunked_amd.workloads import make_inputs_on_device

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LIMIT = 1 << 31
H, K, V = 16, 128, 128
TOL = 2e-2


def rel_l2(x, ref):
    x = x.detach().double().cpu().numpy()
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def stream_slices(g, b, t0, t1, heads):
    """Host copies of rows [t0, t1) of batch row b for the given heads, as
    [1, t1 - t0, len(heads), *] tensors."""
    idx = torch.tensor(heads, device=DEV)
    out = {}
    for n in ("q", "k", "v", "alpha", "beta"):
        x = g[n][b:b + 1, t0:t1].index_select(2, idx)
        out[n] = x.contiguous().cpu()
    return out


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_longest_sequence_at_the_size_limit():
    T = (LIMIT - 1) // (H * max(K, V))          # 1,048,575 tokens
    assert T * H * max(K, V) < LIMIT and T % 64 != 0
    print("case limits: one sequence B=1 T=%d H=%d K=V=%d" % (T, H, K), flush=True)
    g = make_inputs_on_device(1, T, H, K, V, DEV, seed=41)
    o, sf = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], None, chunk=64)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    s = stream_slices(g, 0, 0, T, heads)
    ro, rs = oracle.fwd(s["q"], s["k"], s["v"], s["alpha"], s["beta"], None, nthreads=len(heads))
    idx = torch.tensor(heads, device=DEV)
    eo = rel_l2(o.index_select(2, idx), ro)
    es = rel_l2(sf.index_select(1, idx), rs)
    # the last chunk alone (63 tokens), where the largest offsets are
    el = rel_l2(o[:, T - 63:].index_select(2, idx), ro[:, T - 63:])
    print("  rel L2 o=%.3e final_state=%.3e last chunk=%.3e" % (eo, es, el), flush=True)
    assert np.isfinite(eo) and eo <= TOL and es <= TOL and el <= TOL
    del g, o, sf
    release()


def test_most_streams_at_the_size_limit():
    # the state [B, H, V, K] reaches its cap of 2^31 elements (8.6 GB), the token
    # tensors stay just below theirs; two chunks per sequence, the second ragged
    B = LIMIT // (H * V * K)                     # 8,192 sequences
    T = 127
    assert B * T * H * max(K, V) < LIMIT
    print("case limits: B=%d T=%d H=%d (%d workgroups)" % (B, T, H, B * H * (V // 32)), flush=True)
    g = make_inputs_on_device(B, T, H, K, V, DEV, seed=42)
    o, sf = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], None, chunk=64)
    torch.cuda.synchronize()
    r = np.random.default_rng(42)
    picks = [(0, 0), (B - 1, H - 1)] + [(int(r.integers(B)), int(r.integers(H))) for _ in range(14)]
    for b, h in picks:
        s = stream_slices(g, b, 0, T, [h])
        ro, rs = oracle.fwd(s["q"], s["k"], s["v"], s["alpha"], s["beta"], None, nthreads=1)
        eo = rel_l2(o[b:b + 1, :, h:h + 1], ro)
        es = rel_l2(sf[b:b + 1, h:h + 1], rs)
        assert np.isfinite(eo) and eo <= TOL and es <= TOL, (b, h, eo, es)
    print("  %d sampled streams within %.0e" % (len(picks), TOL), flush=True)
    del g, o, sf
    release()


def test_packed_batch_at_the_size_limit():
    T = (LIMIT - 1) // (H * max(K, V))
    r = np.random.default_rng(43)
    # 64 sequences: a few empty, the rest of random lengths summing to T
    w = r.exponential(1.0, 64)
    w[[5, 17, 40]] = 0.0
    lengths = np.floor(w / w.sum() * T).astype(np.int64)
    lengths[-1] += T - lengths.sum()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    assert cu[-1] == T
    print("case limits: packed batch, %d sequences, %d tokens, H=%d (longest %d)"
          % (len(lengths), T, H, lengths.max()), flush=True)
    g = make_inputs_on_device(1, T, H, K, V, DEV, seed=43)
    o, sf = chunk_fwd_varlen(g["q"], g["k"], g["v"], g["alpha"], g["beta"],
                             torch.from_numpy(cu).to(DEV), None, chunk=64)
    torch.cuda.synchronize()
    for i in range(len(lengths)):
        if lengths[i] == 0:
            assert torch.count_nonzero(sf[i]).item() == 0
    # the shortest non-empty, a middle one and the last sequence (the largest offsets)
    nz = [i for i in range(len(lengths)) if lengths[i] > 0]
    picks = [min(nz, key=lambda i: lengths[i]), nz[len(nz) // 2], nz[-1]]
    for i in picks:
        a, b = int(cu[i]), int(cu[i + 1])
        s = stream_slices(g, 0, a, b, [H - 1])
        ro, rs = oracle.fwd(s["q"], s["k"], s["v"], s["alpha"], s["beta"], None, nthreads=1)
        eo = rel_l2(o[:, a:b, H - 1:H], ro)
        es = rel_l2(sf[i:i + 1, H - 1:H], rs)
        print("  sequence %d (%d tokens at %d): rel L2 o=%.3e state=%.3e" % (i, b - a, a, eo, es),
              flush=True)
        assert np.isfinite(eo) and eo <= TOL and es <= TOL
    del g, o, sf
    release()


# More than 65,536 (batch, head) pairs: every kernel takes a one-dimensional grid,
# since the y and z grid dimensions stop at 65,536 on this GPU.
MANY = 70_000


def test_fp32_forward_and_backward_with_more_than_65536_sequences():
    from linear_attention_sequence_chunked_amd import chunk_bwd
    from linear_attention_sequence_chunked_amd.workloads import make_inputs
    print("case limits: fp32, B=%d T=20 H=1 K=V=16 chunk 16" % MANY, flush=True)
    inp = make_inputs(MANY, 20, 1, 16, 16, dtype=torch.float32, seed=44, gate="decay",
                      s0_std=0.1, with_do=True)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    o, sf = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"], chunk=16)
    got = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], g["initial_state"],
                    chunk=16)
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["initial_state"])
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["d_o"],
                     inp["initial_state"])
    errs = {"o": rel_l2(o, ro), "final_state": rel_l2(sf, rs)}
    for n, x in zip(("dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state"), got):
        errs[n] = rel_l2(x, ref[n])
    print("  " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= 1e-5, (n, e)
    release()


def test_bf16_backward_with_more_than_65536_heads():
    from linear_attention_sequence_chunked_amd import chunk_bwd
    from linear_attention_sequence_chunked_amd.workloads import make_inputs
    print("case limits: bf16 matrix-core backward, B=1 T=64 H=%d K=V=32" % MANY, flush=True)
    inp = make_inputs(1, 64, MANY, 32, 32, dtype=torch.bfloat16, seed=45, gate="decay",
                      with_do=True)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    got = chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"], None, chunk=64)
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["d_o"])
    errs = {n: rel_l2(x, ref[n]) for n, x in zip(("dq", "dk", "dv", "dalpha", "dbeta"), got)}
    print("  " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= TOL, (n, e)
    release()
