"""fp64 CPU oracle of the Kimi Delta Attention (KDA) recurrence -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and the two share no code: the oracle is the plain sequential
recurrence of page "Kimi (AI)", section "Kimi Delta Attention (KDA)" (the
forget-gating / predict / memory-updating equation, with the read-out
o_t = S_t q_t of the linear-attention equation just above it), written in C in
double precision (``kda_oracle.c``).

This module is only argument marshalling: numpy float32 in, numpy float64 out.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE arithmetic, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-Wextra", "-shared", "-fPIC",
           _SRC, "-o", _LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.kda_oracle_prefill_f64.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p, i64p,
                                           i64, i64, i64, i64, f64p, f64p]
    lib.kda_oracle_prefill_f64.restype = ctypes.c_int
    lib.kda_oracle_decode_f64.argtypes = [f32p, f32p, f32p, f32p, f32p,
                                          i64, i64, i64, i64, i64, f64p, f64p]
    lib.kda_oracle_decode_f64.restype = ctypes.c_int
    lib.kda_oracle_prefill_keygate_f64.argtypes = lib.kda_oracle_prefill_f64.argtypes
    lib.kda_oracle_prefill_keygate_f64.restype = ctypes.c_int
    lib.kda_oracle_decode_keygate_f64.argtypes = lib.kda_oracle_decode_f64.argtypes
    lib.kda_oracle_decode_keygate_f64.restype = ctypes.c_int
    lib.kda_oracle_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _f32(x, shape=None):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def prefill(q, k, v, alpha, beta, S0=None, cu_seqlens=None, want_o=True, _key_gate=False):
    """Run the recurrence over packed sequences.

    q, k: [n_tok, H, d_k]; v, alpha: [n_tok, H, d_v]; beta: [n_tok, H]
    S0: [n_seq, H, d_v, d_k] or None (zeros); widened to float64 without change
    cu_seqlens: [n_seq+1] token offsets, or None for one sequence of n_tok tokens.
    Every input must hold exactly the values the GPU receives (bf16 data already
    widened to float32).  Returns (o [n_tok,H,d_v] float64 or None, S_T float64).
    """
    q = np.asarray(q)
    n_tok, H, dk = q.shape
    dv = np.asarray(v).shape[2]
    if cu_seqlens is None:
        cu = np.array([0, n_tok], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n_seq = cu.shape[0] - 1
    if cu[-1] != n_tok:
        raise ValueError("cu_seqlens[-1] must equal n_tok")
    q = _f32(q, (n_tok, H, dk))
    k = _f32(k, (n_tok, H, dk))
    v = _f32(v, (n_tok, H, dv))
    alpha = _f32(alpha, (n_tok, H, dk if _key_gate else dv))
    beta = _f32(beta, (n_tok, H))
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
        if s0.shape != (n_seq, H, dv, dk):
            raise ValueError(f"S0 must be {(n_seq, H, dv, dk)}, got {s0.shape}")
    o = np.empty((n_tok, H, dv), dtype=np.float64) if want_o else None
    ST = np.empty((n_seq, H, dv, dk), dtype=np.float64)
    lib = _load()
    fn = lib.kda_oracle_prefill_keygate_f64 if _key_gate else lib.kda_oracle_prefill_f64
    rc = fn(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(alpha, ctypes.c_float), _ptr(beta, ctypes.c_float),
        None if s0 is None else _ptr(s0, ctypes.c_double), _ptr(cu, ctypes.c_int64),
        n_seq, H, dk, dv,
        None if o is None else _ptr(o, ctypes.c_double), _ptr(ST, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill_f64 failed with code {rc}")
    return o, ST


def decode(q, k, v, alpha, beta, S, want_o=True, _key_gate=False):
    """Run n_steps single-token steps from state S (not modified; a copy is returned).

    q, k: [n_steps, B, H, d_k]; v, alpha: [n_steps, B, H, d_v]; beta: [n_steps, B, H]
    S: [B, H, d_v, d_k].  Returns (o [n_steps,B,H,d_v] float64 or None, S_new float64).
    """
    q = np.asarray(q)
    n_steps, B, H, dk = q.shape
    dv = np.asarray(v).shape[3]
    q = _f32(q)
    k = _f32(k, q.shape)
    v = _f32(v, (n_steps, B, H, dv))
    alpha = _f32(alpha, (n_steps, B, H, dk if _key_gate else dv))
    beta = _f32(beta, (n_steps, B, H))
    Sn = np.array(S, dtype=np.float64, copy=True, order="C")
    if Sn.shape != (B, H, dv, dk):
        raise ValueError("S must be [B, H, d_v, d_k]")
    o = np.empty((n_steps, B, H, dv), dtype=np.float64) if want_o else None
    lib = _load()
    fn = lib.kda_oracle_decode_keygate_f64 if _key_gate else lib.kda_oracle_decode_f64
    rc = fn(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(alpha, ctypes.c_float), _ptr(beta, ctypes.c_float),
        n_steps, B, H, dk, dv, _ptr(Sn, ctypes.c_double),
        None if o is None else _ptr(o, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode_f64 failed with code {rc}")
    return o, Sn


# ------------------------------------------------------- scalar-gate family ---
# The transcript page ("Per dins de Kimi K3 ..."), where it introduces KDA,
# presents it as Gated DeltaNet with the decay control refined to one gate per
# channel.  With one gate per (token, head) the forget step diag(alpha_t) S
# becomes alpha_t S, which is the three-step update above with every row's
# gate equal to alpha_t; no gate at all (the delta rule) is alpha_t = 1.  These
# two functions are that reading written out: they widen the gate to one value
# per value row and run the same recurrence.

def _rows(alpha, lead, dv):
    if alpha is None:
        return np.ones((*lead, dv), dtype=np.float32)
    a = _f32(alpha, lead)
    return np.ascontiguousarray(np.repeat(a[..., None], dv, axis=-1))


def prefill_scalar_gate(q, k, v, alpha, beta, S0=None, cu_seqlens=None, want_o=True):
    """prefill() with alpha [n_tok, H] (one gate per token and head), or None for no gate."""
    v = np.asarray(v)
    return prefill(q, k, v, _rows(alpha, v.shape[:2], v.shape[2]), beta, S0, cu_seqlens, want_o)


def decode_scalar_gate(q, k, v, alpha, beta, S, want_o=True):
    """decode() with alpha [n_steps, B, H] (one gate per step, sequence and head), or None."""
    v = np.asarray(v)
    return decode(q, k, v, _rows(alpha, v.shape[:3], v.shape[3]), beta, S, want_o)


# ------------------------------------------------------- key-channel gate ---
# The forget gate acting on the key side, S~ = S diag(alpha_t) with alpha_t in
# R^{d_k}: the reading of the forget-gating step under which the decay falls on
# key channels; the row form above is the one the section's equations write.

def prefill_key_gate(q, k, v, alpha, beta, S0=None, cu_seqlens=None, want_o=True):
    """prefill() with alpha [n_tok, H, d_k] scaling the columns (key channels) of S."""
    return prefill(q, k, v, alpha, beta, S0, cu_seqlens, want_o, _key_gate=True)


def decode_key_gate(q, k, v, alpha, beta, S, want_o=True):
    """decode() with alpha [n_steps, B, H, d_k] scaling the columns (key channels) of S."""
    return decode(q, k, v, alpha, beta, S, want_o, _key_gate=True)

