"""Pins of the fp64 oracle to facts that the KDA equations fix (CPU only).

Every fact below follows from page "Kimi (AI)", section "Kimi Delta Attention
(KDA)": the forget-gating / predict / memory-updating equation, and the
read-out o_t = S_t q_t of the linear-attention equation of that section.
None of them re-runs the oracle's own loop: they are hand-expanded closed forms,
special cases with a textbook answer, invariants, a hand-worked fixture and an
exact-rational brute force.  Each is chosen so that a plausible slip in the
oracle (decay on columns instead of rows, pre-update read-out, a dropped alpha
in the prediction, a wrong sign of the error, an off-by-one token index) fails
at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(x):
    return np.asarray(x, dtype=np.float32)


def rand_case(rng, T, H, dk, dv, s0=True, alpha_lo=0.3):
    q = f32(rng.standard_normal((T, H, dk)))
    k = f32(rng.standard_normal((T, H, dk)) / np.sqrt(dk))
    v = f32(rng.standard_normal((T, H, dv)))
    a = f32(rng.uniform(alpha_lo, 1.0, (T, H, dv)))
    b = f32(rng.uniform(0.1, 1.0, (T, H)))
    S0 = rng.standard_normal((1, H, dv, dk)) if s0 else None
    return q, k, v, a, b, S0


def d64(x):
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------ worked example
def _read_golden(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = line.split("=", 1)
            vals[key.strip()] = [Fraction(t) for t in rhs.split()]
    return vals


def test_hand_worked_example_d2_t2():
    g = _read_golden("worked_example_d2_t2.txt")
    fl = lambda key, shape: np.array([float(x) for x in g[key]]).reshape(shape)
    q = fl("q", (2, 1, 2))
    k = fl("k", (2, 1, 2))
    v = fl("v", (2, 1, 2))
    a = fl("alpha", (2, 1, 2))
    b = fl("beta", (2, 1))
    S0 = fl("S0", (1, 1, 2, 2))
    o, S = oracle.prefill(q, k, v, a, b, S0)
    # every intermediate is dyadic with few bits: fp64 is exact here
    assert np.array_equal(o, fl("o", (2, 1, 2)))
    assert np.array_equal(S, fl("S_T", (1, 1, 2, 2)))


# ------------------------------------------------------- closed forms, T<=3
def test_T1_closed_form_any_S0():
    rng = np.random.default_rng(1)
    q, k, v, a, b, S0 = rand_case(rng, 1, 3, 5, 4)
    o, S = oracle.prefill(q, k, v, a, b, S0)
    for h in range(3):
        A = d64(a[0, h])[:, None] * S0[0, h]          # rows scaled by alpha_1
        pred = A @ d64(k[0, h])
        S1 = A + b[0, h] * np.outer(d64(v[0, h]) - pred, d64(k[0, h]))
        np.testing.assert_allclose(S[0, h], S1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[0, h], S1 @ d64(q[0, h]), rtol=0, atol=1e-14)


def test_T2_hand_expanded_zero_start():
    rng = np.random.default_rng(2)
    q, k, v, a, b, _ = rand_case(rng, 2, 2, 6, 5, s0=False)
    o, S = oracle.prefill(q, k, v, a, b)
    for h in range(2):
        k1, k2 = d64(k[0, h]), d64(k[1, h])
        q1, q2 = d64(q[0, h]), d64(q[1, h])
        v1, v2 = d64(v[0, h]), d64(v[1, h])
        a2 = d64(a[1, h])
        b1, b2 = float(b[0, h]), float(b[1, h])
        w = a2 * v1                                  # alpha_2 (.) v_1
        e2 = v2 - b1 * (k1 @ k2) * w
        S2 = b1 * np.outer(w, k1) + b2 * np.outer(e2, k2)
        o1 = b1 * (k1 @ q1) * v1
        o2 = b1 * (k1 @ q2) * w + b2 * (k2 @ q2) * e2
        np.testing.assert_allclose(o[0, h], o1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[1, h], o2, rtol=0, atol=1e-14)
        np.testing.assert_allclose(S[0, h], S2, rtol=0, atol=1e-14)


def test_T3_unrolled_rank_one_sum():
    """S_3 = (a3 a2) u1 k1^T + a3 u2 k2^T + u3 k3^T with the hand-unrolled errors."""
    rng = np.random.default_rng(3)
    q, k, v, a, b, _ = rand_case(rng, 3, 2, 7, 3, s0=False)
    o, S = oracle.prefill(q, k, v, a, b)
    for h in range(2):
        K = [d64(k[t, h]) for t in range(3)]
        Q = [d64(q[t, h]) for t in range(3)]
        V = [d64(v[t, h]) for t in range(3)]
        A = [d64(a[t, h]) for t in range(3)]
        B = [float(b[t, h]) for t in range(3)]
        u1 = B[0] * V[0]
        u2 = B[1] * (V[1] - A[1] * u1 * (K[0] @ K[1]))
        u3 = B[2] * (V[2] - A[2] * (A[1] * u1 * (K[0] @ K[2]) + u2 * (K[1] @ K[2])))
        S3 = np.outer(A[2] * A[1] * u1, K[0]) + np.outer(A[2] * u2, K[1]) + np.outer(u3, K[2])
        o1 = u1 * (K[0] @ Q[0])
        o2 = A[1] * u1 * (K[0] @ Q[1]) + u2 * (K[1] @ Q[1])
        o3 = A[2] * A[1] * u1 * (K[0] @ Q[2]) + A[2] * u2 * (K[1] @ Q[2]) + u3 * (K[2] @ Q[2])
        np.testing.assert_allclose(S[0, h], S3, rtol=0, atol=1e-13)
        for t, ot in enumerate((o1, o2, o3)):
            np.testing.assert_allclose(o[t, h], ot, rtol=0, atol=1e-13)


# ----------------------------------------------------------- special cases
def test_alpha_zero_forgets_everything():
    rng = np.random.default_rng(4)
    q, k, v, a, b, S0 = rand_case(rng, 9, 2, 8, 6)
    a[:] = 0.0
    o, S = oracle.prefill(q, k, v, a, b, S0)
    for t in range(9):
        for h in range(2):
            exp_o = float(b[t, h]) * (d64(k[t, h]) @ d64(q[t, h])) * d64(v[t, h])
            np.testing.assert_allclose(o[t, h], exp_o, rtol=0, atol=1e-14)
    for h in range(2):
        np.testing.assert_allclose(S[0, h], float(b[-1, h]) * np.outer(d64(v[-1, h]), d64(k[-1, h])),
                                   rtol=0, atol=1e-14)


def _hadamard(n):
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def test_orthonormal_keys_are_stored_exactly_and_give_linear_attention():
    """alpha=1, beta=1, S0=0, orthonormal keys: S_n k_j = v_j, and the read-out is
    the naive linear attention sum_{s<=t} (k_s . q_t) v_s."""
    d = 16
    keys = _hadamard(d) / 4.0                       # exactly orthonormal rows
    rng = np.random.default_rng(5)
    perm = rng.permutation(d)
    n = 11
    T, H, dv = n, 1, 5
    k = f32(keys[perm[:n]][:, None, :])
    q = f32(rng.standard_normal((T, H, d)))
    v = f32(rng.standard_normal((T, H, dv)))
    a = np.ones((T, H, dv), np.float32)
    b = np.ones((T, H), np.float32)
    o, S = oracle.prefill(q, k, v, a, b)
    for j in range(n):
        np.testing.assert_allclose(S[0, 0] @ d64(k[j, 0]), d64(v[j, 0]), rtol=0, atol=1e-13)
    for t in range(T):
        lin = sum((d64(k[s, 0]) @ d64(q[t, 0])) * d64(v[s, 0]) for s in range(t + 1))
        np.testing.assert_allclose(o[t, 0], lin, rtol=0, atol=1e-13)


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(6)
    q, k, v, a, b, S0 = rand_case(rng, 7, 2, 5, 4)
    b[:] = 0.0
    o, S = oracle.prefill(q, k, v, a, b, S0)
    gam = np.cumprod(d64(a), axis=0)                # gamma_t = prod_{s<=t} alpha_s
    for t in range(7):
        for h in range(2):
            St = gam[t, h][:, None] * S0[0, h]
            np.testing.assert_allclose(o[t, h], St @ d64(q[t, h]), rtol=1e-14, atol=1e-15)
    for h in range(2):
        np.testing.assert_allclose(S[0, h], gam[-1, h][:, None] * S0[0, h], rtol=1e-14, atol=1e-15)


def test_householder_reflections_preserve_frobenius_norm():
    """alpha=1, beta=2, unit k, v=0: S_t = S_{t-1}(I - 2 k k^T), an orthogonal map."""
    rng = np.random.default_rng(7)
    d, T = 8, 12
    k = np.zeros((T, 1, d), np.float32)
    for t in range(T):
        idx = rng.choice(d, 4, replace=False)
        k[t, 0, idx] = 0.5 * rng.choice([-1.0, 1.0], 4)   # exactly unit
    q = f32(rng.standard_normal((T, 1, d)))
    v = np.zeros((T, 1, 6), np.float32)
    a = np.ones((T, 1, 6), np.float32)
    b = np.full((T, 1), 2.0, np.float32)
    S0 = rng.standard_normal((1, 1, 6, d))
    _, S = oracle.prefill(q, k, v, a, b, S0)
    assert abs(np.linalg.norm(S) / np.linalg.norm(S0) - 1.0) < 1e-14
    # and S_T = S0 prod_t (I - 2 k_t k_t^T): reflections on the key side
    R = np.eye(d)
    for t in range(T):
        R = R @ (np.eye(d) - 2.0 * np.outer(d64(k[t, 0]), d64(k[t, 0])))
    np.testing.assert_allclose(S[0, 0], S0[0, 0] @ R, rtol=0, atol=1e-13)


def test_linear_in_v_from_zero_state_and_jointly_in_v_and_S0():
    """S0 = 0: o and S_T are linear in V.  In general they are jointly linear in
    (V, S0) at fixed q, k, alpha, beta.  V is drawn on a 1/64 grid so that the
    combinations are exact float32 values."""
    rng = np.random.default_rng(8)
    q, k, _, a, b, S01 = rand_case(rng, 10, 2, 6, 5)
    v1 = f32(rng.integers(-128, 129, (10, 2, 5)) / 64.0)
    v2 = f32(rng.integers(-128, 129, (10, 2, 5)) / 64.0)
    S02 = rng.standard_normal(S01.shape)
    c1, c2 = 0.75, -1.5
    v12 = f32(c1 * v1 + c2 * v2)
    assert np.array_equal(v12.astype(np.float64), c1 * d64(v1) + c2 * d64(v2))
    o1, S1 = oracle.prefill(q, k, v1, a, b)
    o2, S2 = oracle.prefill(q, k, v2, a, b)
    o12, S12 = oracle.prefill(q, k, v12, a, b)
    np.testing.assert_allclose(o12, c1 * o1 + c2 * o2, rtol=0, atol=1e-13 * np.abs(o12).max())
    np.testing.assert_allclose(S12, c1 * S1 + c2 * S2, rtol=0, atol=1e-13 * np.abs(S12).max())
    o1, S1 = oracle.prefill(q, k, v1, a, b, S01)
    o2, S2 = oracle.prefill(q, k, v2, a, b, S02)
    oS, SS = oracle.prefill(q, k, f32(v1 + v2), a, b, S01 + S02)
    np.testing.assert_allclose(oS, o1 + o2, rtol=0, atol=1e-13 * np.abs(oS).max())
    np.testing.assert_allclose(SS, S1 + S2, rtol=0, atol=1e-13 * np.abs(SS).max())
    # a nonzero start breaks plain linearity in V (the S0 term is not scaled)
    o3, _ = oracle.prefill(q, k, f32(2 * v1), a, b, S01)
    o4, _ = oracle.prefill(q, k, v1, a, b, S01)
    assert np.abs(o3 - 2 * o4).max() > 1e-3


def test_linear_in_v_exact_dyadic():
    """Dyadic inputs keep every product exact, so linearity holds to rounding of sums."""
    rng = np.random.default_rng(9)
    T, d = 6, 4
    k = f32(rng.integers(-4, 5, (T, 1, d)) / 8.0)
    q = f32(rng.integers(-4, 5, (T, 1, d)) / 8.0)
    a = f32(rng.integers(1, 5, (T, 1, d)) / 4.0)
    b = f32(rng.integers(1, 5, (T, 1)) / 4.0)
    v1 = f32(rng.integers(-8, 9, (T, 1, d)) / 8.0)
    v2 = f32(rng.integers(-8, 9, (T, 1, d)) / 8.0)
    o1, S1 = oracle.prefill(q, k, v1, a, b)
    o2, S2 = oracle.prefill(q, k, v2, a, b)
    o3, S3 = oracle.prefill(q, k, f32(v1 + v2), a, b)
    np.testing.assert_allclose(o3, o1 + o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S3, S1 + S2, rtol=0, atol=1e-12)


# --------------------------------------------------- exact rational brute force
def _exact_kda(q, k, v, a, b, S0):
    """Rational arithmetic, written from the three steps as matrix expressions."""
    T, dk = len(k), len(k[0])
    dv = len(v[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        St = [[a[t][i] * S[i][j] for j in range(dk)] for i in range(dv)]
        pred = [sum(St[i][j] * k[t][j] for j in range(dk)) for i in range(dv)]
        S = [[St[i][j] + b[t] * (v[t][i] - pred[i]) * k[t][j] for j in range(dk)] for i in range(dv)]
        outs.append([sum(S[i][j] * q[t][j] for j in range(dk)) for i in range(dv)])
    return outs, S


@pytest.mark.parametrize("seed", [10, 11, 12])
def test_exact_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, dk, dv = 8, 4, 3
    F = lambda x: Fraction(float(x))
    qn = rng.integers(-8, 9, (T, dk)) / 8.0
    kn = rng.integers(-8, 9, (T, dk)) / 16.0
    vn = rng.integers(-16, 17, (T, dv)) / 8.0
    an = rng.integers(0, 9, (T, dv)) / 8.0
    bn = rng.integers(0, 5, (T,)) / 4.0
    S0n = rng.integers(-8, 9, (dv, dk)) / 4.0
    o_ex, S_ex = _exact_kda([[F(x) for x in r] for r in qn], [[F(x) for x in r] for r in kn],
                            [[F(x) for x in r] for r in vn], [[F(x) for x in r] for r in an],
                            [F(x) for x in bn], [[F(x) for x in r] for r in S0n])
    o, S = oracle.prefill(qn[:, None], kn[:, None], vn[:, None], an[:, None], bn[:, None],
                          S0n[None, None])
    o_ref = np.array([[float(x) for x in r] for r in o_ex])
    S_ref = np.array([[float(x) for x in r] for r in S_ex])
    scale = max(np.abs(o_ref).max(), 1.0)
    np.testing.assert_allclose(o[:, 0], o_ref, rtol=0, atol=1e-13 * scale)
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=0, atol=1e-13 * max(np.abs(S_ref).max(), 1.0))


# -------------------------------------------------------------- invariants
def test_value_channel_permutation_and_row_independence():
    rng = np.random.default_rng(13)
    q, k, v, a, b, S0 = rand_case(rng, 12, 2, 6, 7)
    o, S = oracle.prefill(q, k, v, a, b, S0)
    p = rng.permutation(7)
    op, Sp = oracle.prefill(q, k, v[:, :, p], a[:, :, p], b, S0[:, :, p])
    np.testing.assert_array_equal(op, o[:, :, p])
    np.testing.assert_array_equal(Sp, S[:, :, p])
    r = [3]
    o1, S1 = oracle.prefill(q, k, v[:, :, r], a[:, :, r], b, S0[:, :, r])
    np.testing.assert_array_equal(o1, o[:, :, r])
    np.testing.assert_array_equal(S1, S[:, :, r])


def test_equal_rows_reduce_to_scalar_gated_delta_rule():
    """alpha_t = a_t * 1 gives S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    the scalar-gated delta rule (Gated DeltaNet), written here in its key-side
    product form; a_t = 1 gives the plain delta rule.  Checked on the per-channel
    oracle with equal rows and on the scalar-gate entry points (gate [T, H], or
    None for no gate), prefill and decode."""
    rng = np.random.default_rng(14)
    T, dk, dv = 9, 5, 4
    q, k, v, _, b, S0 = rand_case(rng, T, 1, dk, dv)
    for scal in (f32(rng.uniform(0.3, 1.0, T)), np.ones(T, np.float32), None):
        ones = scal is None
        sc = np.ones(T, np.float32) if ones else scal
        a = np.repeat(sc[:, None, None], dv, axis=2).astype(np.float32)
        St = S0[0, 0].copy()
        o_ref = np.zeros((T, dv))
        for t in range(T):
            kt = d64(k[t, 0])
            St = float(sc[t]) * St @ (np.eye(dk) - float(b[t, 0]) * np.outer(kt, kt)) \
                + float(b[t, 0]) * np.outer(d64(v[t, 0]), kt)
            o_ref[t] = St @ d64(q[t, 0])
        runs = [oracle.prefill_scalar_gate(q, k, v, None if ones else sc[:, None], b, S0)]
        dec_o, dec_S = oracle.decode_scalar_gate(q[:, None], k[:, None], v[:, None],
                                                 None if ones else sc[:, None, None], b[:, None], S0)
        runs.append((dec_o[:, 0], dec_S))
        if not ones:
            runs.append(oracle.prefill(q, k, v, a, b, S0))
        for o, S in runs:
            np.testing.assert_allclose(o[:, 0], o_ref, rtol=0, atol=1e-13)
            np.testing.assert_allclose(S[0, 0], St, rtol=0, atol=1e-13)


def test_split_prefill_varlen_and_decode_agree():
    rng = np.random.default_rng(15)
    q, k, v, a, b, S0 = rand_case(rng, 20, 3, 6, 5)
    o, S = oracle.prefill(q, k, v, a, b, S0)
    # split at token 7: continue from the returned fp64 state
    oa, Sa = oracle.prefill(q[:7], k[:7], v[:7], a[:7], b[:7], S0)
    ob, Sb = oracle.prefill(q[7:], k[7:], v[7:], a[7:], b[7:], Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob]), o)
    np.testing.assert_array_equal(Sb, S)
    # varlen: packing three sequences equals running them separately
    lens = [5, 0, 15]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0s = rng.standard_normal((3, 3, 5, 6))
    ov, Sv = oracle.prefill(q, k, v, a, b, S0s, cu)
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        on, Sn = oracle.prefill(q[s:e], k[s:e], v[s:e], a[s:e], b[s:e], S0s[n:n + 1])
        np.testing.assert_array_equal(ov[s:e], on)
        np.testing.assert_array_equal(Sv[n], Sn[0])
    np.testing.assert_array_equal(Sv[1], S0s[1])    # empty sequence: S_T = S0
    # decode over T steps (B=1) equals prefill over T tokens
    od, Sd = oracle.decode(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None], S0[0][None])
    np.testing.assert_array_equal(od[:, 0], o)
    np.testing.assert_array_equal(Sd[0], S[0])


def test_zero_state_default_and_state_only_call():
    rng = np.random.default_rng(16)
    q, k, v, a, b, _ = rand_case(rng, 5, 2, 4, 4, s0=False)
    o1, S1 = oracle.prefill(q, k, v, a, b, None)
    o2, S2 = oracle.prefill(q, k, v, a, b, np.zeros((1, 2, 4, 4)))
    np.testing.assert_array_equal(o1, o2)
    _, S3 = oracle.prefill(q, k, v, a, b, None, want_o=False)
    np.testing.assert_array_equal(S3, S1)


def test_rejects_malformed_cu_seqlens():
    rng = np.random.default_rng(17)
    q, k, v, a, b, _ = rand_case(rng, 6, 1, 4, 4, s0=False)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, a, b, None, np.array([0, 3, 5]))
    with pytest.raises(RuntimeError):
        oracle.prefill(q, k, v, a, b, None, np.array([0, 4, 2, 6]))


def test_segment_composition_identity():
    """The update is affine in the entering state, with the gate on the left (rows) and
    a key-side factor on the right: over any run of tokens
        S_end = diag(Gamma) S_start M + dS,
    where Gamma is the product of the gates per row, M is what the recurrence makes of
    S_start = I with v = 0 and no gate, and dS is the run from S_start = 0.  Composing
    the runs of consecutive segments reproduces the whole sequence (the identity the
    sequence-parallel prefill relies on), for uneven segment lengths."""
    rng = np.random.default_rng(16)
    T, dk, dv = 23, 5, 5
    q, k, v, a, b, S0 = rand_case(rng, T, 1, dk, dv)
    _, S_whole = oracle.prefill(q, k, v, a, b, S0)
    S = S0[0, 0].copy()
    for s, e in ((0, 7), (7, 8), (8, 19), (19, 23)):
        sl = slice(s, e)
        _, dS = oracle.prefill(q[sl], k[sl], v[sl], a[sl], b[sl], None)
        _, M = oracle.prefill(q[sl], k[sl], np.zeros_like(v[sl]), np.ones_like(a[sl]), b[sl],
                              np.eye(dk)[None, None])
        gamma = np.prod(d64(a[sl, 0]), axis=0)
        S = gamma[:, None] * (S @ M[0, 0]) + dS[0, 0]
    np.testing.assert_allclose(S, S_whole[0, 0], rtol=0, atol=1e-12)


# ------------------------------------------------ key-channel gate (S~ = S diag(alpha))
def key_case(rng, T, H, dk, dv):
    q, k, v, _, b, S0 = rand_case(rng, T, H, dk, dv)
    a = f32(rng.uniform(0.3, 1.0, (T, H, dk)))
    return q, k, v, a, b, S0


def test_key_gate_T1_closed_form():
    """S_1 = S0 diag(alpha_1) + beta_1 (v_1 - S0 diag(alpha_1) k_1) k_1^T, o_1 = S_1 q_1."""
    rng = np.random.default_rng(21)
    q, k, v, a, b, S0 = key_case(rng, 1, 1, 4, 3)
    St = S0[0, 0] * d64(a[0, 0])[None, :]
    S1 = St + float(b[0, 0]) * np.outer(d64(v[0, 0]) - St @ d64(k[0, 0]), d64(k[0, 0]))
    o, S = oracle.prefill_key_gate(q, k, v, a, b, S0)
    np.testing.assert_allclose(S[0, 0], S1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 0], S1 @ d64(q[0, 0]), rtol=0, atol=1e-14)


def test_key_gate_T2_from_zero_decays_the_key_side():
    """From S0 = 0: S_1 = b1 v1 k1^T and
    S_2 = b1 v1 (a2 * k1)^T + b2 (v2 - b1 ((a2 * k1) . k2) v1) k2^T: the gate multiplies the
    stored key, where the row form would multiply the stored value."""
    rng = np.random.default_rng(22)
    q, k, v, a, b, _ = key_case(rng, 2, 1, 4, 3)
    k1, k2, v1, v2 = d64(k[0, 0]), d64(k[1, 0]), d64(v[0, 0]), d64(v[1, 0])
    a2, b1, b2 = d64(a[1, 0]), float(b[0, 0]), float(b[1, 0])
    ak1 = a2 * k1
    S2 = b1 * np.outer(v1, ak1) + b2 * np.outer(v2 - b1 * (ak1 @ k2) * v1, k2)
    o, S = oracle.prefill_key_gate(q, k, v, a, b, None)
    np.testing.assert_allclose(S[0, 0], S2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[1, 0], S2 @ d64(q[1, 0]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 0], b1 * (k1 @ d64(q[0, 0])) * v1, rtol=0, atol=1e-14)


def test_key_gate_equal_channels_is_the_scalar_gate_and_zero_forgets():
    """A gate equal on every key channel scales S as a whole, like the scalar gate (and the
    row form with equal rows); alpha = 0 forgets everything: S_t = beta_t v_t k_t^T."""
    rng = np.random.default_rng(23)
    q, k, v, _, b, S0 = key_case(rng, 11, 2, 5, 4)
    sc = f32(rng.uniform(0.3, 1.0, (11, 2)))
    o1, S1 = oracle.prefill_key_gate(q, k, v, np.repeat(sc[..., None], 5, axis=2), b, S0)
    o2, S2 = oracle.prefill_scalar_gate(q, k, v, sc, b, S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-13)
    o3, S3 = oracle.prefill_key_gate(q, k, v, np.zeros((11, 2, 5), np.float32), b, S0)
    exp_S = d64(b[-1])[:, None, None] * d64(v[-1])[:, :, None] * d64(k[-1])[:, None, :]
    np.testing.assert_allclose(S3[0], exp_S, rtol=0, atol=1e-14)
    exp_o = (d64(b) * (d64(k) * d64(q)).sum(-1))[..., None] * d64(v)
    np.testing.assert_allclose(o3, exp_o, rtol=0, atol=1e-14)


def test_key_gate_key_channel_permutation():
    """Permuting key channels (q, k, alpha and the columns of S0) permutes the columns of
    S_T and leaves o unchanged; decode over the steps is the prefill."""
    rng = np.random.default_rng(24)
    q, k, v, a, b, S0 = key_case(rng, 9, 1, 6, 3)
    p = rng.permutation(6)
    o, S = oracle.prefill_key_gate(q, k, v, a, b, S0)
    op, Sp = oracle.prefill_key_gate(q[..., p], k[..., p], v, a[..., p], b, S0[..., p])
    np.testing.assert_allclose(op, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sp, S[..., p], rtol=0, atol=1e-13)
    od, Sd = oracle.decode_key_gate(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None], S0)
    np.testing.assert_allclose(od[:, 0], o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sd, S, rtol=0, atol=1e-13)
