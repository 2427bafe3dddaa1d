"""Python binding of libkda: the C ABI of include/kda.h, one function per entry point.

Argument marshalling only -- every step of the computation runs in the HIP
kernels of libkda.so.  Tensors are torch tensors on the GPU (PyTorch provides
device memory and the current stream); there is no CPU fallback, and a missing
library raises at first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_DEVICE = 3
KDA_ERR_WORKSPACE = 4
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1

EXPORTED = ("kda_abi_version", "kda_status_string", "kda_prefill_workspace_size", "kda_prefill",
            "kda_decode_step", "kda_prefill_scalar_gate", "kda_decode_step_scalar_gate",
            "kda_prefill_key_gate", "kda_decode_step_key_gate", "kda_prefill_backward_workspace_size",
            "kda_prefill_backward", "kda_prefill_backward_scalar_gate", "kda_prefill_backward_key_gate",
            "kda_prefill_noalloc", "kda_prefill_key_gate_workspace_size")
NOALLOC_MAX_WORKSPACE = 256 << 20  # KDA_PREFILL_NOALLOC_MAX_WORKSPACE

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libkda.so with argument types set (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkda.so not found at {LIB_PATH}; build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.kda_abi_version.restype = ctypes.c_int
    L.kda_abi_version.argtypes = []
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_prefill_workspace_size.restype = sz
    L.kda_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    L.kda_prefill_key_gate_workspace_size.restype = sz
    L.kda_prefill_key_gate_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    for name in ("kda_prefill", "kda_prefill_scalar_gate", "kda_prefill_key_gate"):
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                       vp, vp, vp, sz, vp]
    for name in ("kda_decode_step", "kda_decode_step_scalar_gate", "kda_decode_step_key_gate"):
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, vp]
    L.kda_prefill_noalloc.restype = ctypes.c_int
    L.kda_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp, vp, vp]
    L.kda_prefill_backward_workspace_size.restype = sz
    L.kda_prefill_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    for name in ("kda_prefill_backward", "kda_prefill_backward_scalar_gate", "kda_prefill_backward_key_gate"):
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                       vp, vp, vp, vp, vp, vp, vp, sz, vp]
    _lib = L
    return L


def abi_version() -> int:
    return lib().kda_abi_version()


def status_string(status: int) -> str:
    return lib().kda_status_string(status).decode()


def workspace_size(n_seq: int, n_tok: int, n_heads: int, d_k: int, d_v: int, dtype_code: int) -> int:
    return int(lib().kda_prefill_workspace_size(n_seq, n_tok, n_heads, d_k, d_v, dtype_code))


def key_gate_workspace_size(n_seq: int, n_tok: int, n_heads: int, d_k: int, d_v: int, dtype_code: int) -> int:
    return int(lib().kda_prefill_key_gate_workspace_size(n_seq, n_tok, n_heads, d_k, d_v, dtype_code))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libkda takes GPU tensors only")
    if not t.is_contiguous():
        raise ValueError("libkda takes contiguous tensors only")
    return t.data_ptr()


def _expect(name, t, shape, dtype):
    """Raise ValueError unless tensor t (may not be None) has this shape and dtype."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _gate_shape(fn: str, n_tok: int, H: int, dk: int, dv: int):
    """Shape of alpha for the gate form of entry point fn (None: the form takes none)."""
    if fn.endswith("_key_gate"):
        return (n_tok, H, dk)
    if fn.endswith("_scalar_gate"):
        return (n_tok, H)
    return (n_tok, H, dv)


def _check_qkv(q, k, v):
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be 3-d: [n_tok, H, d_k], [n_tok, H, d_k], [n_tok, H, d_v]")
    _dtype_code(q)
    _expect("k", k, q.shape, q.dtype)
    if v.shape[:2] != q.shape[:2] or v.dtype != q.dtype:
        raise ValueError(f"v must be [{q.shape[0]}, {q.shape[1]}, d_v] in {q.dtype}, got "
                         f"{tuple(v.shape)} {v.dtype}")
    return torch


def _check_inputs(fn, q, k, v, alpha, beta, S0, n_seq):
    """Shapes and dtypes of a prefill call's inputs (the C ABI sees raw pointers only)."""
    torch = _check_qkv(q, k, v)
    n_tok, H, dk = q.shape
    dv = v.shape[2]
    f32 = torch.float32
    if alpha is not None or not fn.endswith("_scalar_gate"):
        _expect("alpha", alpha, _gate_shape(fn, n_tok, H, dk, dv), f32)
    _expect("beta", beta, (n_tok, H), f32)
    if S0 is not None:
        _expect("S0", S0, (n_seq, H, dv, dk), f32)


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def kda_prefill(q, k, v, alpha, beta, S0=None, cu_seqlens=None, *, n_seq: Optional[int] = None,
                o=None, S_T=None, want_state: bool = True, workspace=None):
    """Chunkwise KDA prefill over packed sequences.

    q, k: [n_tok, H, d_k]; v: [n_tok, H, d_v] (bf16 or f32, same dtype)
    alpha: [n_tok, H, d_v] f32; beta: [n_tok, H] f32
    S0: [n_seq, H, d_v, d_k] f32 or None (zeros)
    cu_seqlens: int32 [n_seq+1] on the GPU, or None with n_seq equal sequences
    (n_seq defaults to 1).  Returns (o, S_T); S_T is None if want_state is
    False.  S_T may be passed as S0 for an in-place continuation.
    """
    return _prefill("kda_prefill", q, k, v, alpha, beta, S0, cu_seqlens, n_seq, o, S_T, want_state,
                    workspace)


def kda_prefill_scalar_gate(q, k, v, alpha, beta, S0=None, cu_seqlens=None, *,
                            n_seq: Optional[int] = None, o=None, S_T=None, want_state: bool = True,
                            workspace=None):
    """Prefill with one forget gate per (token, head) for every row (Gated DeltaNet):
    alpha is [n_tok, H] f32, or None for no gate (alpha = 1, the delta rule).  The
    other arguments and the result are those of kda_prefill."""
    return _prefill("kda_prefill_scalar_gate", q, k, v, alpha, beta, S0, cu_seqlens, n_seq, o, S_T,
                    want_state, workspace)


def kda_prefill_key_gate(q, k, v, alpha, beta, S0=None, cu_seqlens=None, *,
                         n_seq: Optional[int] = None, o=None, S_T=None, want_state: bool = True,
                         workspace=None):
    """Prefill with the forget gate on key channels (S~ = S diag(alpha)): alpha is
    [n_tok, H, d_k] f32.  The other arguments and the result are those of kda_prefill."""
    return _prefill("kda_prefill_key_gate", q, k, v, alpha, beta, S0, cu_seqlens, n_seq, o, S_T,
                    want_state, workspace)


def _prefill(fn, q, k, v, alpha, beta, S0, cu_seqlens, n_seq, o, S_T, want_state, workspace):
    torch = _check_qkv(q, k, v)
    n_tok, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-d int32 tensor")
        n_seq = cu_seqlens.shape[0] - 1
    elif n_seq is None:
        n_seq = S0.shape[0] if S0 is not None else 1
    _check_inputs(fn, q, k, v, alpha, beta, S0, n_seq)
    if o is None:
        o = torch.empty((n_tok, H, dv), dtype=q.dtype, device=q.device)
    _expect("o", o, (n_tok, H, dv), q.dtype)
    if S_T is None and want_state:
        S_T = torch.empty((n_seq, H, dv, dk), dtype=torch.float32, device=q.device)
    if S_T is not None:
        _expect("S_T", S_T, (n_seq, H, dv, dk), torch.float32)
    size_fn = key_gate_workspace_size if fn == "kda_prefill_key_gate" else workspace_size
    ws_bytes = size_fn(n_seq, n_tok, H, dk, dv, dt)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
                            _ptr(cu_seqlens), n_seq, n_tok, H, dk, dv, dt, _ptr(o), _ptr(S_T),
                            _ptr(workspace), 0 if workspace is None else workspace.numel(),
                            _stream(q))
    if st != KDA_OK:
        raise KdaError(fn, st)
    return o, S_T


def kda_prefill_noalloc(q, k, v, alpha, beta, S0=None, cu_seqlens=None, *, n_seq: Optional[int] = None,
                        o=None, S_T=None, want_state: bool = True):
    """kda_prefill with the library's own device workspace (no workspace argument, nothing
    allocated by the library call).  o and S_T are allocated here unless given; callers that
    cannot allocate pass them.  Same arguments and result as kda_prefill."""
    torch = _check_qkv(q, k, v)
    n_tok, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-d int32 tensor")
        n_seq = cu_seqlens.shape[0] - 1
    elif n_seq is None:
        n_seq = S0.shape[0] if S0 is not None else 1
    _check_inputs("kda_prefill", q, k, v, alpha, beta, S0, n_seq)
    if o is None:
        o = torch.empty((n_tok, H, dv), dtype=q.dtype, device=q.device)
    _expect("o", o, (n_tok, H, dv), q.dtype)
    if S_T is None and want_state:
        S_T = torch.empty((n_seq, H, dv, dk), dtype=torch.float32, device=q.device)
    if S_T is not None:
        _expect("S_T", S_T, (n_seq, H, dv, dk), torch.float32)
    st = lib().kda_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
                                   n_seq, n_tok, H, dk, dv, _dtype_code(q), _ptr(o), _ptr(S_T), _stream(q))
    if st != KDA_OK:
        raise KdaError("kda_prefill_noalloc", st)
    return o, S_T


def kda_decode_step(q, k, v, alpha, beta, S, o=None):
    """One decode step for every (sequence, head): S is updated in place.

    q, k: [B, H, d_k]; v: [B, H, d_v]; alpha: [B, H, d_v] f32; beta: [B, H] f32;
    S: [B, H, d_v, d_k] f32.  Returns o [B, H, d_v] in q's dtype.
    """
    return _decode("kda_decode_step", q, k, v, alpha, beta, S, o)


def kda_decode_step_scalar_gate(q, k, v, alpha, beta, S, o=None):
    """Decode step with one forget gate per (sequence, head) for every row: alpha is
    [B, H] f32, or None for no gate (the delta rule).  Otherwise as kda_decode_step."""
    return _decode("kda_decode_step_scalar_gate", q, k, v, alpha, beta, S, o)


def kda_decode_step_key_gate(q, k, v, alpha, beta, S, o=None):
    """Decode step with the forget gate on key channels: alpha is [B, H, d_k] f32.
    Otherwise as kda_decode_step."""
    return _decode("kda_decode_step_key_gate", q, k, v, alpha, beta, S, o)


def _decode(fn, q, k, v, alpha, beta, S, o):
    torch = _check_qkv(q, k, v)
    B, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if alpha is not None or not fn.endswith("_scalar_gate"):
        _expect("alpha", alpha, _gate_shape(fn, B, H, dk, dv), torch.float32)
    _expect("beta", beta, (B, H), torch.float32)
    _expect("S", S, (B, H, dv, dk), torch.float32)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _expect("o", o, (B, H, dv), q.dtype)
    st = getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S), _ptr(o),
                            B, H, dk, dv, dt, _stream(q))
    if st != KDA_OK:
        raise KdaError(fn, st)
    return o


def backward_workspace_size(n_seq: int, n_tok: int, n_heads: int, d_k: int, d_v: int) -> int:
    return int(lib().kda_prefill_backward_workspace_size(n_seq, n_tok, n_heads, d_k, d_v))


def _backward(fn, q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq, want_dS0, workspace):
    torch = _check_qkv(q, k, v)
    n_tok, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-d int32 tensor")
        n_seq = cu_seqlens.shape[0] - 1
    elif n_seq is None:
        n_seq = S0.shape[0] if S0 is not None else 1
    _check_inputs(fn.replace("_backward", ""), q, k, v, alpha, beta, S0, n_seq)
    # the incoming gradients are float32 whatever the input dtype (o of a bf16 call is bf16)
    _expect("dO", dO, (n_tok, H, dv), torch.float32)
    if dS_T is not None:
        _expect("dS_T", dS_T, (n_seq, H, dv, dk), torch.float32)
    f32 = dict(dtype=torch.float32, device=q.device)
    grads = dict(dq=torch.empty((n_tok, H, dk), **f32), dk=torch.empty((n_tok, H, dk), **f32),
                 dv=torch.empty((n_tok, H, dv), **f32),
                 dalpha=None if alpha is None else torch.empty(alpha.shape, **f32),
                 dbeta=torch.empty((n_tok, H), **f32),
                 dS0=torch.empty((n_seq, H, dv, dk), **f32) if want_dS0 else None)
    ws_bytes = backward_workspace_size(n_seq, n_tok, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
                            _ptr(dO), _ptr(dS_T), n_seq, n_tok, H, dk, dv, _dtype_code(q),
                            _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dalpha"]),
                            _ptr(grads["dbeta"]), _ptr(grads["dS0"]), _ptr(workspace), workspace.numel(),
                            _stream(q))
    if st != KDA_OK:
        raise KdaError(fn, st)
    return grads


def kda_prefill_backward(q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T=None, *, n_seq: Optional[int] = None,
                         want_dS0: bool = True, workspace=None):
    """Gradients (dict dq, dk, dv, dalpha, dbeta, dS0; float32) of a kda_prefill call's
    inputs, given dO = dL/do (float32 [n_tok, H, d_v]) and dS_T = dL/dS_T (or None)."""
    return _backward("kda_prefill_backward", q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq, want_dS0,
                     workspace)


def kda_prefill_backward_scalar_gate(q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T=None, *,
                                     n_seq: Optional[int] = None, want_dS0: bool = True, workspace=None):
    """kda_prefill_backward with alpha [n_tok, H] (one gate per token and head) or None (no gate)."""
    return _backward("kda_prefill_backward_scalar_gate", q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq,
                     want_dS0, workspace)


def kda_prefill_backward_key_gate(q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T=None, *,
                                  n_seq: Optional[int] = None, want_dS0: bool = True, workspace=None):
    """kda_prefill_backward with the gate on key channels, alpha [n_tok, H, d_k]."""
    return _backward("kda_prefill_backward_key_gate", q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq,
                     want_dS0, workspace)
