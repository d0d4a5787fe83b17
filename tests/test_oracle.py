"""Pins of the fp64 token oracle against facts the mathematics fixes.

None of these re-types the oracle's loop: each checks a closed form, an
invariant or an independent formulation, chosen so that a plausible slip in the
oracle (a dropped alpha or beta, the wrong read order, a transposed state, a
gate index off by one) fails at least one of them.

Facts used (from the pages, restated):
  * token order: decay, read with k from the decayed state, write beta times the
    error, then read the output with q from the UPDATED state ("Sparse Delta
    Memory: layer and kernels", "What the layer computes"; dense limit in
    "Product-key top-k");
  * state layout [B,H,V,K] and exact streaming continuation ("OpenGDN 0.1.0",
    "Core operator reference");
  * chunking changes results only by rounding ("Sparse Delta Memory", same
    section, paragraph after the chunk steps).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.chunk_algebra import chunked_forward


def _rand(rng, B, T, H, K, V, unit_k=True, s0=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    a = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, V, K)) if s0 else None
    return q, k, v, a, b, S0


def test_zero_gate_zero_state_gives_zero_output():
    # alpha = 1, beta = 0 and a zero state: nothing is ever written, so o == 0 exactly.
    rng = np.random.default_rng(0)
    q, k, v, _, _, _ = _rand(rng, 2, 37, 3, 8, 5)
    o, sf = oracle.fwd(q, k, v, np.ones((2, 37, 3)), np.zeros((2, 37, 3)))
    assert np.all(o == 0.0) and np.all(sf == 0.0)


def test_identity_gates_read_initial_state():
    # alpha = 1, beta = 0: the state never changes, o_t = S0 q_t (row-major [V,K] layout).
    rng = np.random.default_rng(1)
    B, T, H, K, V = 2, 11, 3, 6, 4
    q, k, v, _, _, S0 = _rand(rng, B, T, H, K, V)
    o, sf = oracle.fwd(q, k, v, np.ones((B, T, H)), np.zeros((B, T, H)), S0)
    expect = np.einsum("bhvk,bthk->bthv", S0, q)
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(sf, S0)


def test_pure_decay_is_product_of_gates():
    # beta = 0: S_t = (prod_{s<=t} alpha_s) S0 and o_t = gamma_t S0 q_t (gate index pinned).
    rng = np.random.default_rng(2)
    B, T, H, K, V = 1, 20, 2, 5, 7
    q, k, v, a, _, S0 = _rand(rng, B, T, H, K, V)
    o, sf = oracle.fwd(q, k, v, a, np.zeros((B, T, H)), S0)
    gam = np.cumprod(a, axis=1)  # [B,T,H]
    expect = gam[..., None] * np.einsum("bhvk,bthk->bthv", S0, q)
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sf, gam[:, -1][..., None, None] * S0, rtol=1e-12)


def test_unit_beta_unit_key_writes_value_exactly():
    # beta = 1 and |k_t| = 1: S_t k_t = v_t for every t.  With q = k the output
    # (read from the UPDATED state) is therefore v_t itself.
    rng = np.random.default_rng(3)
    B, T, H, K, V = 2, 30, 2, 8, 6
    _, k, v, a, _, S0 = _rand(rng, B, T, H, K, V)
    o, sf = oracle.fwd(k, k, v, a, np.ones((B, T, H)), S0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.einsum("bhvk,bhk->bhv", sf, k[:, -1]), v[:, -1], atol=1e-12)


def test_orthonormal_keys_update_one_column():
    # k_t = e_{j_t}: S (I - b e_j e_j^T) zeroes column j, so column j becomes
    # a(1-b) S[:, j] + b v_t and every other column becomes a S[:, c].  K != V
    # checks the [V, K] orientation.
    rng = np.random.default_rng(4)
    B, T, H, K, V = 1, 15, 1, 5, 3
    q = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    a = rng.uniform(0.3, 1.0, (B, T, H))
    b = rng.uniform(0.0, 1.0, (B, T, H))
    idx = rng.integers(0, K, T)
    k = np.zeros((B, T, H, K))
    k[0, np.arange(T), 0, idx] = 1.0
    S0 = rng.standard_normal((B, H, V, K))
    o, sf = oracle.fwd(q, k, v, a, b, S0)
    S = S0[0, 0].copy()
    for t in range(T):
        j, at, bt = idx[t], a[0, t, 0], b[0, t, 0]
        col = at * (1.0 - bt) * S[:, j] + bt * v[0, t, 0]
        S = at * S
        S[:, j] = col
        np.testing.assert_allclose(o[0, t, 0], S @ q[0, t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sf[0, 0], S, rtol=1e-12, atol=1e-12)


def test_single_token_matrix_form():
    # T = 1 written as a matrix product: S1 = a S0 (I - b k k^T) + b v k^T, o = S1 q.
    rng = np.random.default_rng(5)
    B, H, K, V = 2, 3, 7, 4
    q, k, v, a, b, S0 = _rand(rng, B, 1, H, K, V, unit_k=False)
    o, sf = oracle.fwd(q, k, v, a, b, S0)
    for bb in range(B):
        for hh in range(H):
            kk, vv, qq = k[bb, 0, hh], v[bb, 0, hh], q[bb, 0, hh]
            S1 = a[bb, 0, hh] * S0[bb, hh] @ (np.eye(K) - b[bb, 0, hh] * np.outer(kk, kk)) \
                + b[bb, 0, hh] * np.outer(vv, kk)
            np.testing.assert_allclose(sf[bb, hh], S1, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(o[bb, 0, hh], S1 @ qq, rtol=1e-13, atol=1e-13)


def test_hand_worked_two_token_example():
    # K = V = 2, S0 = 0.
    # t=1: k=e1, v=(1,2), a=1/2, b=1/2 -> S1 = 1/2 v k^T = [[.5,0],[1,0]]; q=(1,1) -> o=(.5,1)
    # t=2: k=e2, v=(-1,4), a=1/4, b=1 -> S2 = 1/4 S1 (I - e2 e2^T) + v e2^T = [[.125,-1],[.25,4]]
    #      q=(2,-1) -> o = (0.25+1, 0.5-4) = (1.25, -3.5)
    k = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    v = np.array([[1.0, 2.0], [-1.0, 4.0]]).reshape(1, 2, 1, 2)
    q = np.array([[1.0, 1.0], [2.0, -1.0]]).reshape(1, 2, 1, 2)
    a = np.array([0.5, 0.25]).reshape(1, 2, 1)
    b = np.array([0.5, 1.0]).reshape(1, 2, 1)
    o, sf = oracle.fwd(q, k, v, a, b)
    np.testing.assert_array_equal(o[0, :, 0], [[0.5, 1.0], [1.25, -3.5]])
    np.testing.assert_array_equal(sf[0, 0], [[0.125, -1.0], [0.25, 4.0]])


def test_streaming_continuation_is_exact():
    # Two calls carrying final_state equal one call, bit for bit in fp64.
    rng = np.random.default_rng(6)
    B, T, H, K, V = 2, 50, 2, 6, 5
    q, k, v, a, b, S0 = _rand(rng, B, T, H, K, V)
    o, sf = oracle.fwd(q, k, v, a, b, S0)
    cut = 23
    o1, s1 = oracle.fwd(q[:, :cut], k[:, :cut], v[:, :cut], a[:, :cut], b[:, :cut], S0)
    o2, s2 = oracle.fwd(q[:, cut:], k[:, cut:], v[:, cut:], a[:, cut:], b[:, cut:], s1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(s2, sf)


def test_linear_in_values_and_initial_state():
    # For fixed q, k, alpha, beta the map (v, S0) -> (o, S_T) is linear, and o is linear in q.
    rng = np.random.default_rng(7)
    B, T, H, K, V = 1, 40, 2, 6, 6
    q, k, v1, a, b, S01 = _rand(rng, B, T, H, K, V)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    c1, c2 = 0.7, -1.3
    o1, s1 = oracle.fwd(q, k, v1, a, b, S01)
    o2, s2 = oracle.fwd(q, k, v2, a, b, S02)
    o3, s3 = oracle.fwd(q, k, c1 * v1 + c2 * v2, a, b, c1 * S01 + c2 * S02)
    np.testing.assert_allclose(o3, c1 * o1 + c2 * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, c1 * s1 + c2 * s2, rtol=1e-11, atol=1e-12)
    q2 = rng.standard_normal(q.shape)
    oa, _ = oracle.fwd(q2, k, v1, a, b, S01)
    ob, _ = oracle.fwd(q + q2, k, v1, a, b, S01)
    np.testing.assert_allclose(ob, o1 + oa, rtol=1e-11, atol=1e-12)


def _exact_forward(q, k, v, a, b):
    # Exact rational arithmetic, token order decay -> read -> write -> read output.
    T, K = len(q), len(q[0])
    V = len(v[0])
    M = [[Fraction(0)] * K for _ in range(V)]  # state [V, K]
    outs = []
    for t in range(T):
        M = [[a[t] * x for x in row] for row in M]
        r = [sum(M[i][c] * k[t][c] for c in range(K)) for i in range(V)]
        M = [[M[i][c] + b[t] * (v[t][i] - r[i]) * k[t][c] for c in range(K)] for i in range(V)]
        outs.append([sum(M[i][c] * q[t][c] for c in range(K)) for i in range(V)])
    return outs, M


def test_fp64_rounding_against_exact_rationals():
    # The oracle's only deviation from the exact result is fp64 rounding.
    rng = np.random.default_rng(8)
    T, K, V = 6, 3, 4

    def rat(shape, den):
        return rng.integers(-den, den + 1, shape) / den
    q, k, v = rat((T, K), 8), rat((T, K), 8), rat((T, V), 8)
    a = rng.integers(1, 9, T) / 8
    b = rng.integers(0, 9, T) / 8
    F = lambda x: [[Fraction(float(y)) for y in row] for row in x]  # noqa: E731
    outs, M = _exact_forward(F(q), F(k), F(v), [Fraction(float(x)) for x in a],
                             [Fraction(float(x)) for x in b])
    o, sf = oracle.fwd(q[None, :, None], k[None, :, None], v[None, :, None],
                       a[None, :, None], b[None, :, None])
    np.testing.assert_allclose(o[0, :, 0], np.array(outs, dtype=np.float64), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(sf[0, 0], np.array(M, dtype=np.float64), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_chunk_algebra_matches_token_oracle(chunk):
    # The extended-WY chunk steps reach the token result up to rounding, for any
    # chunk size and a ragged last chunk, from a nonzero state.
    rng = np.random.default_rng(9)
    B, T, H, K, V = 2, 150, 2, 16, 12
    q, k, v, _, b, S0 = _rand(rng, B, T, H, K, V)
    a = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((B, T, H)))))
    o, sf = oracle.fwd(q, k, v, a, b, S0)
    oc, sc = chunked_forward(q, k, v, a, b, S0, chunk=chunk)
    assert np.linalg.norm(oc - o) / np.linalg.norm(o) < 1e-12
    assert np.linalg.norm(sc - sf) / np.linalg.norm(sf) < 1e-12


def test_threads_do_not_change_bits():
    rng = np.random.default_rng(10)
    q, k, v, a, b, S0 = _rand(rng, 3, 40, 3, 8, 8)
    o1, s1 = oracle.fwd(q, k, v, a, b, S0, nthreads=1)
    o4, s4 = oracle.fwd(q, k, v, a, b, S0, nthreads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(s1, s4)
