"""Pins of the backward oracle (oracle.backward.prefill_backward) against things other
than itself: central finite differences of the forward oracle (itself pinned in
test_oracle_pins), and a closed form for one token from a zero state.

Inputs are dyadic (multiples of 2^-6) so that x +- 2^-12 is exact in float32, the
forward oracle's input type; it computes in float64, so the central difference is
off from the derivative only by its O(eps^2) truncation term."""
import numpy as np
import pytest

import oracle
from oracle.backward import prefill_backward

EPS = 2.0 ** -12


def dyadic(rng, shape, lo, hi):
    return (np.round(rng.uniform(lo, hi, size=shape) * 64) / 64).astype(np.float32)


def make_case(seed, lens, H, dk, dv, gate):
    rng = np.random.default_rng(seed)
    n = sum(lens)
    c = dict(q=dyadic(rng, (n, H, dk), -1, 1), k=dyadic(rng, (n, H, dk), -0.7, 0.7),
             v=dyadic(rng, (n, H, dv), -1, 1), beta=dyadic(rng, (n, H), 0.1, 0.9),
             S0=dyadic(rng, (len(lens), H, dv, dk), -0.5, 0.5).astype(np.float64),
             dO=rng.standard_normal((n, H, dv)), dS_T=rng.standard_normal((len(lens), H, dv, dk)),
             cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))
    c["alpha"] = {"channel": dyadic(rng, (n, H, dv), 0.5, 1.0), "scalar": dyadic(rng, (n, H), 0.5, 1.0),
                  "none": None, "key": dyadic(rng, (n, H, dk), 0.5, 1.0)}[gate]
    return c


def loss(c, gate):
    fwd = {"channel": oracle.prefill, "scalar": oracle.prefill_scalar_gate, "none": oracle.prefill_scalar_gate,
           "key": oracle.prefill_key_gate}[gate]
    o, S = fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["S0"], c["cu"])
    return float((o * c["dO"]).sum() + (S * c["dS_T"]).sum())


@pytest.mark.parametrize("gate", ["channel", "scalar", "none", "key"])
def test_backward_matches_central_differences_of_the_forward(gate):
    c = make_case(11, [4, 0, 3], 2, 4, 3, gate)
    g = prefill_backward(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["S0"], c["cu"], c["dO"], c["dS_T"], gate)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("S0", "dS0")]
    if gate != "none":
        names.append(("alpha", "dalpha"))
    for x, dx in names:
        base = c[x]
        fd = np.zeros(base.shape)
        for idx in np.ndindex(base.shape):
            keep = base[idx]
            base[idx] = keep + EPS
            lp = loss(c, gate)
            base[idx] = keep - EPS
            lm = loss(c, gate)
            base[idx] = keep
            fd[idx] = (lp - lm) / (2 * EPS)
        scale = max(1.0, np.abs(fd).max())
        np.testing.assert_allclose(g[dx], fd, rtol=0, atol=2e-6 * scale, err_msg=f"{gate}: {dx}")
    if gate == "none":
        assert g["dalpha"] is None


def test_backward_one_token_zero_state_closed_form():
    # o = beta (k.q) v and S_1 = beta v k^T, so with L = dO.o + <dS_T, S_1>:
    # dv = beta ((k.q) dO + dS_T k), dbeta = (k.q)(v.dO) + v^T dS_T k,
    # dq = beta (v.dO) k, dk = beta ((v.dO) q + dS_T^T v), dalpha = 0 (the state was zero),
    # dS0 = diag(alpha) (dS_T + dO q^T) - beta alpha (.) (dS_T k + (k.q) dO) k^T
    rng = np.random.default_rng(5)
    dk, dv = 5, 3
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    al, b = rng.uniform(0.2, 1.0, dv), 0.6
    dO, dST = rng.standard_normal(dv), rng.standard_normal((dv, dk))
    g = prefill_backward(q[None, None], k[None, None], v[None, None], al[None, None], np.array([[b]]), None,
                         [0, 1], dO[None, None], dST[None, None], "channel")
    kq, vdo = k @ q, v @ dO
    np.testing.assert_allclose(g["dv"][0, 0], b * (kq * dO + dST @ k), rtol=1e-13)
    np.testing.assert_allclose(g["dbeta"][0, 0], kq * vdo + v @ dST @ k, rtol=1e-13)
    np.testing.assert_allclose(g["dq"][0, 0], b * vdo * k, rtol=1e-13)
    np.testing.assert_allclose(g["dk"][0, 0], b * (vdo * q + dST.T @ v), rtol=1e-13)
    np.testing.assert_allclose(g["dalpha"][0, 0], np.zeros(dv), atol=1e-15)
    du = dST @ k + kq * dO
    np.testing.assert_allclose(g["dS0"][0, 0], al[:, None] * (dST + np.outer(dO, q)) - np.outer(b * al * du, k),
                               rtol=1e-12, atol=1e-14)


def test_backward_of_a_scalar_gate_sums_the_row_gradients():
    c = make_case(12, [6], 1, 4, 3, "scalar")
    rows = np.repeat(c["alpha"][:, :, None], 3, axis=2)
    gs = prefill_backward(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["S0"], c["cu"], c["dO"], c["dS_T"], "scalar")
    gc = prefill_backward(c["q"], c["k"], c["v"], rows, c["beta"], c["S0"], c["cu"], c["dO"], c["dS_T"], "channel")
    np.testing.assert_allclose(gs["dalpha"], gc["dalpha"].sum(axis=2), rtol=1e-13)
    for x in ("dq", "dk", "dv", "dbeta", "dS0"):
        np.testing.assert_array_equal(gs[x], gc[x])
