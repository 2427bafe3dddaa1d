"""fp64 CPU oracle of the KDA recurrence's gradients -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library never does.

Page "Kimi (AI)", section "Kimi Delta Attention (KDA)": per token the state
S (d_v x d_k, rows = value channels) goes through three steps, and the
read-out uses the updated state:
    forget:   S~ = diag(alpha_t) S_{t-1}
    predict:  v~ = S~ k_t           ( = alpha_t (.) a_t with a_t = S_{t-1} k_t )
    update:   S_t = S~ + beta_t (v_t - v~) k_t^T      ( u_t = beta_t (v_t - v~) )
    read-out: o_t = S_t q_t
The transcript page ("Per dins de Kimi K3 ..."), where it turns to training,
says the model is trained with the chunk-wise parallel algorithm, which needs
these gradients.  For a scalar loss L with dL/do_t = dO_t and dL/dS_T = dS_T, the
chain rule taken through the steps in reverse order, token by token, with
G_t = dL/dS_t (everything that depends on S_t) is:
    G_t      = (gradient flowing from S_{t+1}) + dO_t q_t^T
    dq_t     = S_t^T dO_t
    du_t     = G_t k_t
    dk_t     = G_t^T u_t + S_{t-1}^T da_t,          da_t = -beta_t alpha_t (.) du_t
    dv_t     = beta_t du_t
    dbeta_t  = du_t . (v_t - alpha_t (.) a_t)
    dalpha_t = rowsum(G_t (.) S_{t-1}) - beta_t a_t (.) du_t
    dL/dS_{t-1} = diag(alpha_t) G_t + da_t k_t^T
and dS0 = dL/dS_{-1} after the first token.  A gate shared by all rows (one
scalar per token and head) receives the sum of dalpha_t over the rows; no
gate (alpha = 1) has no alpha gradient.
With the gate on key channels instead, S~ = S_{t-1} diag(alpha_t) (alpha_t in
R^{d_k}), a_t = S~ k_t, u_t = beta_t (v_t - a_t), S_t = S~ + u_t k_t^T:
    G_t      = (gradient flowing from S_{t+1}) + dO_t q_t^T,   dq_t = S_t^T dO_t
    du_t     = G_t k_t,  da_t = -beta_t du_t,  dv_t = beta_t du_t,
    dbeta_t  = du_t . (v_t - a_t),  dk_t = G_t^T u_t + S~^T da_t,
    dS~      = G_t + da_t k_t^T,
    dalpha_t = colsum(dS~ (.) S_{t-1})           (one value per key channel)
    dL/dS_{-1+t} = dS~ diag(alpha_t).  The states S_{t-1} are kept from a
plain forward pass.  Plain numpy, per (sequence, head), one token at a time.
Pinned in tests by central finite differences of the forward oracle.
"""
from __future__ import annotations

import numpy as np


def prefill_backward(q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T=None, gate="channel"):
    """Gradients of L = sum(dO * o) + sum(dS_T * S_T) for one prefill call.

    q, k: [n_tok, H, d_k]; v, dO: [n_tok, H, d_v]; beta: [n_tok, H];
    alpha: [n_tok, H, d_v] (gate "channel"), [n_tok, H] ("scalar"), None ("none") or
    [n_tok, H, d_k] ("key": the gate on key channels);
    S0, dS_T: [n_seq, H, d_v, d_k] or None (zeros); cu_seqlens: [n_seq + 1].
    Returns dict with dq, dk, dv, dalpha (None for "none"), dbeta, dS0 (float64).
    """
    f = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    q, k, v, beta, dO, S0, dS_T = f(q), f(k), f(v), f(beta), f(dO), f(S0), f(dS_T)
    n_tok, H, dk_ = q.shape
    dv_ = v.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n_seq = cu.shape[0] - 1
    if gate == "key":
        return _backward_key_gate(q, k, v, f(alpha), beta, S0, cu, dO, dS_T)
    if gate == "channel":
        a_rows = f(alpha)
    elif gate == "scalar":
        a_rows = np.repeat(f(alpha)[:, :, None], dv_, axis=2)
    elif gate == "none":
        a_rows = np.ones((n_tok, H, dv_))
    else:
        raise ValueError(gate)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dbeta=np.zeros((n_tok, H)),
               dS0=np.zeros((n_seq, H, dv_, dk_)))
    dalpha_rows = np.zeros((n_tok, H, dv_))
    for n in range(n_seq):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S = np.zeros((dv_, dk_)) if S0 is None else S0[n, h].copy()
            states = [S]                      # states[i] = state before token s + i
            for t in range(s, e):
                al, kt, vt, bt = a_rows[t, h], k[t, h], v[t, h], beta[t, h]
                a = S @ kt
                u = bt * (vt - al * a)
                S = al[:, None] * S + np.outer(u, kt)
                states.append(S)
            G_next = np.zeros((dv_, dk_)) if dS_T is None else dS_T[n, h].copy()
            for t in range(e - 1, s - 1, -1):
                Sp, St = states[t - s], states[t - s + 1]
                al, kt, qt, vt, bt, dOt = a_rows[t, h], k[t, h], q[t, h], v[t, h], beta[t, h], dO[t, h]
                a = Sp @ kt
                u = bt * (vt - al * a)
                G = G_next + np.outer(dOt, qt)
                out["dq"][t, h] = St.T @ dOt
                du = G @ kt
                da = -bt * al * du
                out["dk"][t, h] = G.T @ u + Sp.T @ da
                out["dv"][t, h] = bt * du
                out["dbeta"][t, h] = du @ (vt - al * a)
                dalpha_rows[t, h] = (G * Sp).sum(axis=1) - bt * a * du
                G_next = al[:, None] * G + np.outer(da, kt)
            out["dS0"][n, h] = G_next
    out["dalpha"] = (dalpha_rows if gate == "channel" else dalpha_rows.sum(axis=2) if gate == "scalar"
                     else None)
    return out


def _backward_key_gate(q, k, v, alpha, beta, S0, cu, dO, dS_T):
    n_tok, H, dk_ = q.shape
    dv_ = v.shape[2]
    n_seq = cu.shape[0] - 1
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dalpha=np.zeros_like(alpha),
               dbeta=np.zeros((n_tok, H)), dS0=np.zeros((n_seq, H, dv_, dk_)))
    for n in range(n_seq):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S = np.zeros((dv_, dk_)) if S0 is None else S0[n, h].copy()
            states = [S]
            for t in range(s, e):
                St = S * alpha[t, h][None, :]
                u = beta[t, h] * (v[t, h] - St @ k[t, h])
                S = St + np.outer(u, k[t, h])
                states.append(S)
            G_next = np.zeros((dv_, dk_)) if dS_T is None else dS_T[n, h].copy()
            for t in range(e - 1, s - 1, -1):
                Sp, Snew = states[t - s], states[t - s + 1]
                al, kt, qt, vt, bt, dOt = alpha[t, h], k[t, h], q[t, h], v[t, h], beta[t, h], dO[t, h]
                St = Sp * al[None, :]
                a = St @ kt
                u = bt * (vt - a)
                G = G_next + np.outer(dOt, qt)
                out["dq"][t, h] = Snew.T @ dOt
                du = G @ kt
                da = -bt * du
                out["dv"][t, h] = bt * du
                out["dbeta"][t, h] = du @ (vt - a)
                out["dk"][t, h] = G.T @ u + St.T @ da
                dSt = G + np.outer(da, kt)
                out["dalpha"][t, h] = (dSt * Sp).sum(axis=0)
                G_next = dSt * al[None, :]
            out["dS0"][n, h] = G_next
    return out
