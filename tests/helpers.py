"""Shared test helpers: parity metrics, tolerances and host->device upload.

Parity metric (per (sequence, head) slice, separately for o and S_T):
    max_rel = max|gpu - ref| / max|ref|      rms_rel = ||gpu - ref||_2 / ||ref||_2
Element-wise relative error is undefined near zero, so the norm-wise form is used.
"""
from __future__ import annotations

import numpy as np

# float32 inputs: fp32 arithmetic in the GPU path against the fp64 oracle
TOL_F32 = dict(max_rel=1e-4, rms_rel=1e-4)
# bf16 inputs (oracle fed the same bf16 values), o rounded to bf16
TOL_BF16 = dict(max_rel=1e-2, rms_rel=3e-3)


def tol_for(dtype: str) -> dict:
    return TOL_F32 if dtype == "f32" else TOL_BF16


def rel_errors(gpu: np.ndarray, ref: np.ndarray):
    d = gpu.astype(np.float64) - ref
    den_max = np.abs(ref).max()
    den_rms = np.sqrt((ref * ref).sum())
    if den_max == 0.0:
        return (0.0 if np.abs(d).max() == 0 else np.inf), (0.0 if np.abs(d).max() == 0 else np.inf)
    return float(np.abs(d).max() / den_max), float(np.sqrt((d * d).sum()) / den_rms)


def worst_slices(gpu: np.ndarray, ref: np.ndarray, slices):
    """Worst (max_rel, rms_rel) over an iterable of index tuples into gpu/ref."""
    wmax = wrms = 0.0
    for sl in slices:
        m, r = rel_errors(gpu[sl], ref[sl])
        wmax, wrms = max(wmax, m), max(wrms, r)
    return wmax, wrms


def check(name: str, gpu: np.ndarray, ref: np.ndarray, slices, tol: dict):
    m, r = worst_slices(gpu, ref, slices)
    gm, gr = rel_errors(gpu, ref)
    msg = f"{name}: worst slice max_rel={m:.3e} rms_rel={r:.3e}; global max_rel={gm:.3e} rms_rel={gr:.3e}"
    print(msg, flush=True)
    assert m <= tol["max_rel"] and r <= tol["rms_rel"], msg + f" exceeds {tol}"
    return m, r


def o_slices(cu, H, seqs=None, heads=None):
    """Index tuples of o [n_tok, H, d_v] for each (sequence, head) pair."""
    seqs = range(len(cu) - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    return [(slice(int(cu[n]), int(cu[n + 1])), h) for n in seqs for h in heads
            if cu[n + 1] > cu[n]]


def s_slices(n_seq, H):
    return [(n, h) for n in range(n_seq) for h in range(H)]


# ------------------------------------------------------------------ device
def to_device(x: np.ndarray, dtype: str, device="cuda"):
    """Host array -> GPU tensor; bf16 data arrives as uint16 bit patterns."""
    import torch
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def from_device(t) -> np.ndarray:
    """GPU tensor -> float64 numpy (bf16 widened exactly)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def upload_prefill(inp, device="cuda"):
    import torch
    d = dict(
        q=to_device(inp.q, inp.dtype, device), k=to_device(inp.k, inp.dtype, device),
        v=to_device(inp.v, inp.dtype, device),
        alpha=None if inp.alpha is None else to_device(inp.alpha, "f32", device),
        beta=to_device(inp.beta, "f32", device),
        S0=None if inp.S0 is None else to_device(inp.S0, "f32", device),
        cu_seqlens=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device),
    )
    return d


def oracle_prefill_subset(inp, seqs, heads, rows=None):
    """Oracle on chosen sequences/heads (and optionally value rows) only.

    Heads and value rows are independent in the recurrence (rows because the
    gate is a per-row scalar), so a subset reproduces those outputs exactly.
    Returns dict (seq, head) -> (o [len, d_v'], S_T [d_v', d_k]).
    """
    import oracle
    out = {}
    rows = slice(None) if rows is None else rows
    for n in seqs:
        s, e = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        hs = list(heads)
        q = inp.f32("q")[s:e][:, hs] if e > s else np.zeros((0, len(hs), inp.dk), np.float32)
        k = inp.f32("k")[s:e][:, hs]
        v = inp.f32("v")[s:e][:, hs][:, :, rows]
        a = inp.alpha[s:e][:, hs][:, :, rows]
        b = inp.beta[s:e][:, hs]
        S0 = None if inp.S0 is None else inp.S0[n:n + 1][:, hs][:, :, rows].astype(np.float64)
        o, S = oracle.prefill(q, k, v, a, b, S0)
        for j, h in enumerate(hs):
            out[(n, h)] = (o[:, j], S[0, j])
    return out
