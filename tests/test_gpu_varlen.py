"""Packed variable-length forward (gdn_chunk_fwd_varlen) through the C ABI.

Each packed sequence must equal the fp64 oracle run on that sequence alone from
its own initial state (1e-5 float32 / 2e-2 bfloat16 relative L2), equal-length
packing must reproduce the dense call bitwise, and an empty sequence must hand
its initial state through unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunked_amd import chunk_fwd, chunk_fwd_varlen
from linear_attention_sequence_chunked_amd.workloads import make_inputs

from tests.parity import assert_parity, worst_local

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
DEV = torch.device("cuda:0")


def rel_l2(x, ref):
    x = x.detach().double().cpu().numpy()
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def packed(lengths, H, K, V, dt, seed, chunk_dt=None):
    """One input set per sequence (own seed), packed along T; returns (parts, packed dict, cu)."""
    parts = [make_inputs(1, max(L, 1), H, K, V, dtype=dt, seed=seed + i, s0_std=0.05)
             for i, L in enumerate(lengths)]
    for p, L in zip(parts, lengths):
        for n in ("q", "k", "v", "alpha", "beta"):
            p[n] = p[n][:, :L].contiguous()
    cat = {n: torch.cat([p[n] for p in parts], 1) for n in ("q", "k", "v", "alpha", "beta")}
    cat["initial_state"] = torch.cat([p["initial_state"] for p in parts], 0)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return parts, cat, cu


@pytest.mark.parametrize("dt,K,V,chunk", [(torch.bfloat16, 128, 128, 64), (torch.float32, 64, 32, 32),
                                          (torch.bfloat16, 64, 128, 32), (torch.bfloat16, 32, 32, 16)])
def test_ragged_batch_matches_per_sequence_oracle(dt, K, V, chunk):
    lengths = [1, 17, 64, 65, 200, 0, 333, 128]
    print("case varlen %s K=%d V=%d chunk=%d lengths=%s" % (dt, K, V, chunk, lengths), flush=True)
    parts, cat, cu = packed(lengths, 3, K, V, dt, seed=500 + K + V)
    g = {n: t.to(DEV) for n, t in cat.items()}
    o, sf = chunk_fwd_varlen(g["q"], g["k"], g["v"], g["alpha"], g["beta"], cu.to(DEV),
                             g["initial_state"], chunk=chunk)
    torch.cuda.synchronize()
    for i, (p, L) in enumerate(zip(parts, lengths)):
        s0 = p["initial_state"]
        if L == 0:
            assert torch.equal(sf[i].cpu(), s0[0]), "empty sequence must keep its state"
            continue
        ro, rs = oracle.fwd(p["q"], p["k"], p["v"], p["alpha"], p["beta"], s0)
        a, b = int(cu[i]), int(cu[i + 1])
        print("  seq %d L=%d" % (i, L), flush=True)
        assert_parity("seq %d" % i, {"o": (o[:, a:b], ro), "final_state": (sf[i:i + 1], rs)}, TOL[dt])


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_equal_lengths_reproduce_dense_call_bitwise(dt):
    B, T, H = 3, 150, 2
    inp = make_inputs(B, T, H, 64, 64, dtype=dt, seed=77, s0_std=0.05)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in inp.items()}
    C = 64 if dt == torch.bfloat16 else 32
    od, sd = chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["initial_state"], chunk=C)
    flat = {n: g[n].reshape((1, B * T) + tuple(g[n].shape[2:])).contiguous()
            for n in ("q", "k", "v", "alpha", "beta")}
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device=DEV)
    ov, sv = chunk_fwd_varlen(flat["q"], flat["k"], flat["v"], flat["alpha"], flat["beta"], cu,
                              g["initial_state"], chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(ov.reshape(od.shape), od)
    assert torch.equal(sv, sd)


# Workgroup scheduling of the bf16 kernel depends on the batch shape: (sequence,
# head) pairs spread over the XCDs when they divide by 8, a plain id order when the
# workgroups do not, a contiguous run per XCD otherwise; sequences start longest
# first for up to 128 of them.  Every path must give each sequence its own result.
SCHEDULE_CASES = [
    # (lengths, H, K, V)
    ([70, 5, 300, 64, 129], 1, 64, 32),                   # 10 workgroups: id order, longest first
    ([90, 90, 7, 250, 250, 33], 2, 64, 128),               # 96 workgroups, 12 pairs: contiguous runs
    ([40, 40, 40, 3, 3, 160, 160, 1], 1, 32, 32),          # equal lengths: ties in table order
    ([(7 * i) % 61 + 1 for i in range(136)], 1, 32, 32),   # 136 sequences: spread, table order
]


@pytest.mark.parametrize("case", SCHEDULE_CASES, ids=lambda c: "n%dH%dK%dV%d" % (len(c[0]), c[1], c[2], c[3]))
def test_ragged_schedule_paths(case):
    lengths, H, K, V = case
    print("case varlen schedule n=%d H=%d K=%d V=%d" % (len(lengths), H, K, V), flush=True)
    parts, cat, cu = packed(lengths, H, K, V, torch.bfloat16, seed=900 + len(lengths))
    g = {n: t.to(DEV) for n, t in cat.items()}
    o, sf = chunk_fwd_varlen(g["q"], g["k"], g["v"], g["alpha"], g["beta"], cu.to(DEV),
                             g["initial_state"], chunk=64)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (p, L) in enumerate(zip(parts, lengths)):
        ro, rs = oracle.fwd(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["initial_state"])
        a, b = int(cu[i]), int(cu[i + 1])
        eo, es = rel_l2(o[:, a:b], ro), rel_l2(sf[i:i + 1], rs)
        worst = max(worst, eo, es)
        assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16], (i, L, eo, es)
        for name, x, ref in (("o", o[:, a:b], ro), ("final_state", sf[i:i + 1], rs)):
            wb, at = worst_local(name, x, ref)
            worst = max(worst, wb)
            assert wb <= TOL[torch.bfloat16], (i, L, name, wb, at)
    print("  worst rel L2 (whole or block) %.2e" % worst, flush=True)


def test_reset_mask_as_packed_sequences():
    # rows of a [B, T] batch with resets (state set to zero before the token):
    # boundaries at every row start and reset, the row's own initial state for
    # its first piece and zeros for the others; each row's final state is its
    # last piece's.  The oracle runs every piece on its own.
    B, T, H, K, V = 3, 400, 2, 64, 64
    inp = make_inputs(B, T, H, K, V, dtype=torch.bfloat16, seed=650, s0_std=0.05)
    r = np.random.default_rng(651)
    reset = r.random((B, T)) < 0.01
    reset[:, 0] = False
    starts, s0, last = [], [], []
    for b in range(B):
        cuts = [0] + [int(t) for t in np.nonzero(reset[b])[0]]
        for j, c in enumerate(cuts):
            starts.append(b * T + c)
            s0.append(inp["initial_state"][b] if j == 0 else torch.zeros(H, V, K))
        last.append(len(starts) - 1)
    cu = torch.tensor(starts + [B * T], dtype=torch.int32)
    flat = {n: inp[n].reshape((1, B * T) + tuple(inp[n].shape[2:])).contiguous()
            for n in ("q", "k", "v", "alpha", "beta")}
    print("case reset mask: %d pieces from %d resets" % (len(starts), int(reset.sum())), flush=True)
    g = {n: t.to(DEV) for n, t in flat.items()}
    o, sf = chunk_fwd_varlen(g["q"], g["k"], g["v"], g["alpha"], g["beta"], cu.to(DEV),
                             torch.stack(s0).to(DEV), chunk=64)
    torch.cuda.synchronize()
    for i in range(len(starts)):
        a, e = int(cu[i]), int(cu[i + 1])
        piece = {n: flat[n][:, a:e] for n in flat}
        ro, rs = oracle.fwd(piece["q"], piece["k"], piece["v"], piece["alpha"], piece["beta"],
                            s0[i].unsqueeze(0))
        assert rel_l2(o[:, a:e], ro) <= TOL[torch.bfloat16], i
        assert worst_local("o", o[:, a:e], ro)[0] <= TOL[torch.bfloat16], i
        if i in last:
            assert rel_l2(sf[i:i + 1], rs) <= TOL[torch.bfloat16], i
