"""The chunk algebra the GPU prefill uses, in float64 numpy, against the oracle.

Within a chunk of tokens (state S entering it), with G[t,i] = sum_{s<=t} log alpha[s,i]:
    L = strictly_lower(diag(beta) K K^T),  A = (I + L)^{-1} diag(beta)
    U = A (V * e^{-G} - K S^T)
    O = e^{G} * (Q S^T + tril(Q K^T) U)
    S' = diag(e^{G[-1,:]}) (S + U^T K)
This is the three-step update of page "Kimi (AI)", section "Kimi Delta Attention (KDA)",
regrouped: the gate scales state rows, so it commutes with everything on the key side and the
decayed Gram of row i is D_i L D_i^{-1}.  Padding a partial chunk with k=q=v=0, beta=0,
alpha=1 tokens must change nothing.
"""
import numpy as np
import pytest

import oracle


def chunk_prefill(q, k, v, a, b, S0, C, pad_to_chunk=False):
    T, dk = q.shape
    dv = v.shape[1]
    S = S0.copy()
    O = np.zeros((T, dv))
    for c0 in range(0, T, C):
        Q, K, V, Al, B = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C], a[c0:c0 + C], b[c0:c0 + C]
        n = len(Q)
        if pad_to_chunk and n < C:
            pad = C - n
            Q = np.vstack([Q, np.zeros((pad, dk))])
            K = np.vstack([K, np.zeros((pad, dk))])
            V = np.vstack([V, np.zeros((pad, dv))])
            Al = np.vstack([Al, np.ones((pad, dv))])
            B = np.concatenate([B, np.zeros(pad)])
        m = len(Q)
        G = np.cumsum(np.log(Al), axis=0)
        L = np.tril(B[:, None] * (K @ K.T), -1)
        A = np.linalg.solve(np.eye(m) + L, np.diag(B))
        U = A @ (V * np.exp(-G) - K @ S.T)
        Oc = np.exp(G) * (Q @ S.T + np.tril(Q @ K.T) @ U)
        S = np.exp(G[-1])[:, None] * (S + U.T @ K)
        O[c0:c0 + n] = Oc[:n]
    return O, S


def case(seed, T, dk, dv, alpha_lo=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = rng.uniform(alpha_lo, 1.0, (T, dv))
    b = rng.uniform(0.05, 1.0, T)
    S0 = 0.02 * rng.standard_normal((dv, dk))
    f = lambda x: np.asarray(x, np.float32).astype(np.float64)  # values the oracle takes exactly
    return f(q), f(k), f(v), f(a), f(b), S0


@pytest.mark.parametrize("C", [1, 2, 16, 64, 100])
def test_chunk_form_matches_recurrence(C):
    q, k, v, a, b, S0 = case(C, 256, 64, 48)
    o_ref, S_ref = oracle.prefill(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None],
                                  S0[None, None])
    O, S = chunk_prefill(q, k, v, a, b, S0, C)
    np.testing.assert_allclose(O, o_ref[:, 0], rtol=0, atol=1e-12 * np.abs(o_ref).max())
    np.testing.assert_allclose(S, S_ref[0, 0], rtol=0, atol=1e-12 * np.abs(S_ref).max())


@pytest.mark.parametrize("T", [1, 63, 65, 130])
def test_padded_partial_chunk_is_exact(T):
    q, k, v, a, b, S0 = case(100 + T, T, 32, 16)
    o_ref, S_ref = oracle.prefill(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None],
                                  S0[None, None])
    O, S = chunk_prefill(q, k, v, a, b, S0, 64, pad_to_chunk=True)
    np.testing.assert_allclose(O, o_ref[:, 0], rtol=0, atol=1e-12 * np.abs(o_ref).max())
    np.testing.assert_allclose(S, S_ref[0, 0], rtol=0, atol=1e-12 * np.abs(S_ref).max())


def test_decay_free_solve_equals_per_row_decayed_solves():
    """(I + D L D^{-1})^{-1} = D (I + L)^{-1} D^{-1}: one solve serves every row."""
    rng = np.random.default_rng(7)
    C = 16
    K = rng.standard_normal((C, 8)) / np.sqrt(8)
    beta = rng.uniform(0.1, 1, C)
    L = np.tril(beta[:, None] * (K @ K.T), -1)
    g = np.cumsum(np.log(rng.uniform(0.5, 1, C)))
    D = np.diag(np.exp(g))
    lhs = np.linalg.inv(np.eye(C) + D @ L @ np.linalg.inv(D))
    rhs = D @ np.linalg.inv(np.eye(C) + L) @ np.linalg.inv(D)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
