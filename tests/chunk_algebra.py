"""fp64 numpy statement of the extended-WY / UT chunk decomposition (test helper).

This is NOT the oracle (the oracle is the token loop in ``oracle/``).  It writes
out, in float64 and one chunk at a time, the chunk algebra the HIP kernels follow,
so the tests can check that derivation against the token oracle independently of
any GPU.  The steps are those "Sparse Delta Memory: layer and kernels" lists in
"What the layer computes" (cumulative log-decays, the decay-weighted Gram
matrices A (strictly causal) and QK (causal), the solve X = (I + tril(beta A,
-1))^-1, then a sequential state pass), specialised to the dense case, and the
extended-WY form named by "OpenGDN 0.1.0" ("Core operator reference").

For one stream and one chunk of n tokens with chunk-start state S [V,K]:
    g_r   = sum_{i<=r} ln alpha_i,     gam = exp(g)
    A_ri  = beta_r exp(g_r - g_i) k_r.k_i   (i < r),  0 otherwise
    P_ri  = exp(g_r - g_i) q_r.k_i          (i <= r), 0 otherwise
    Tm    = (I + A)^-1
    W     = Tm diag(beta gam) K,   Ut = Tm diag(beta) Vc
    U     = Ut - W S^T
    O     = diag(gam) Q S^T + P U
    S'    = gam_n S + U^T diag(gam_n / gam) K
"""
import numpy as np


def chunked_forward(q, k, v, alpha, beta, s0=None, chunk=64):
    q, k, v, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    o = np.zeros((B, T, H, V))
    sf = np.zeros((B, H, V, K))
    for b in range(B):
        for h in range(H):
            S = np.zeros((V, K)) if s0 is None else np.array(s0[b, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                Q, Kc, Vc = q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h]
                al, be = alpha[b, t0:t1, h], beta[b, t0:t1, h]
                n = t1 - t0
                g = np.cumsum(np.log(al))
                gam = np.exp(g)
                diff = g[:, None] - g[None, :]
                lower_strict = np.tril(np.ones((n, n), dtype=bool), -1)
                lower = np.tril(np.ones((n, n), dtype=bool), 0)
                dec = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
                A = np.where(lower_strict, be[:, None] * dec * (Kc @ Kc.T), 0.0)
                P = np.where(lower, dec * (Q @ Kc.T), 0.0)
                Tm = np.linalg.inv(np.eye(n) + A)
                W = Tm @ ((be * gam)[:, None] * Kc)
                Ut = Tm @ (be[:, None] * Vc)
                U = Ut - W @ S.T
                o[b, t0:t1, h] = gam[:, None] * (Q @ S.T) + P @ U
                S = gam[-1] * S + U.T @ ((gam[-1] / gam)[:, None] * Kc)
            sf[b, h] = S
    return o, sf
