"""Pins of the oracle's reverse mode (the hand-derived VJP of the token loop).

Checked two derivation-independent ways, the layered strategy that "atomic_ops
0.1.0" describes under "Correctness & testing": central finite differences of the
fp64 forward oracle, and float64 autograd through an independent torch token loop
(matrix form S = a S (I - b k k^T) + b v k^T).
"""
import numpy as np
import torch

import oracle


def _inputs(seed, B=1, T=9, H=2, K=4, V=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    a = rng.uniform(0.5, 1.0, (B, T, H))
    b = rng.uniform(0.1, 0.9, (B, T, H))
    S0 = rng.standard_normal((B, H, V, K))
    dO = rng.standard_normal((B, T, H, V))
    dSf = rng.standard_normal((B, H, V, K))
    return dict(q=q, k=k, v=v, alpha=a, beta=b, initial_state=S0), dO, dSf


def _loss(inp, dO, dSf):
    o, sf = oracle.fwd(**inp)
    return float(np.sum(o * dO) + np.sum(sf * dSf))


def test_reverse_matches_central_differences():
    inp, dO, dSf = _inputs(0)
    g = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dO,
                   inp["initial_state"], dSf)
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta",
             "initial_state": "d_initial_state"}
    rng = np.random.default_rng(1)
    eps = 1e-6
    for name, gname in names.items():
        x = inp[name]
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(inp, dO, dSf)
            x[idx] = old - eps
            lm = _loss(inp, dO, dSf)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[gname][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[gname][idx])


def _torch_token_loop(q, k, v, a, b, S0):
    B, T, H, K = q.shape
    V = v.shape[-1]
    outs = []
    S = S0
    eye = torch.eye(K, dtype=torch.float64)
    for t in range(T):
        kt = k[:, t]  # [B,H,K]
        proj = eye - b[:, t, :, None, None] * kt[..., :, None] * kt[..., None, :]
        S = a[:, t, :, None, None] * (S @ proj) + b[:, t, :, None, None] * v[:, t, ..., :, None] * kt[..., None, :]
        outs.append((S @ q[:, t, ..., None])[..., 0])
    return torch.stack(outs, dim=1), S


def test_reverse_matches_float64_autograd():
    inp, dO, dSf = _inputs(2, B=2, T=70, H=2, K=5, V=4)  # crosses the 64-token checkpoint
    t = {n: torch.tensor(x, requires_grad=True) for n, x in inp.items()}
    o, sf = _torch_token_loop(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["initial_state"])
    loss = (o * torch.tensor(dO)).sum() + (sf * torch.tensor(dSf)).sum()
    loss.backward()
    g = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dO,
                   inp["initial_state"], dSf)
    # the torch loop is also a second, independent statement of the forward
    o_ref, sf_ref = oracle.fwd(**inp)
    np.testing.assert_allclose(o.detach().numpy(), o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sf.detach().numpy(), sf_ref, rtol=1e-12, atol=1e-12)
    pairs = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta",
             "initial_state": "d_initial_state"}
    for n, gn in pairs.items():
        np.testing.assert_allclose(g[gn], t[n].grad.numpy(), rtol=1e-10, atol=1e-10, err_msg=n)


def test_output_gradient_identity():
    # dq_t = S_t^T dO_t: with d_final_state = 0 and dO nonzero only at token t,
    # dq_t is the updated state transposed times dO_t (checked against a forward call).
    inp, dO, _ = _inputs(3, T=12)
    t = 7
    dOt = np.zeros_like(dO)
    dOt[:, t] = dO[:, t]
    g = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dOt, inp["initial_state"])
    _, S_t = oracle.fwd(*(inp[n][:, : t + 1] for n in ("q", "k", "v", "alpha", "beta")),
                        initial_state=inp["initial_state"])
    np.testing.assert_allclose(g["dq"][:, t], np.einsum("bhvk,bhv->bhk", S_t, dO[:, t]), rtol=1e-12)
    assert np.all(g["dq"][:, t + 1:] == 0.0)
