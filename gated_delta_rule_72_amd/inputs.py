"""Seeded synthetic inputs for the KDA prefill and decode workloads.

This module holds random draws, dtype rounding and shapes only -- none of the
recurrence's arithmetic -- so that the GPU path and the fp64 oracle can be fed
identical bits from one place.

Recipe (every draw is independent; see also ``WORKLOADS``):
  * Each tensor is drawn in blocks along its leading (token or step) axis;
    a block holds max(1, 2**22 // E) leading entries, E being the element
    count of one entry.  Block b of tensor number n uses its own generator
    ``Generator(PCG64(SeedSequence([seed, n, b])))``, so blocks can be drawn
    in parallel threads and the result does not depend on thread count.
  * q, k: N(0, 1) per element in float64, L2-normalised per (token, head)
    vector in float64, then rounded to the input dtype (bf16 round-to-nearest-
    even, or float32).
  * v: N(0, 1), rounded the same way.
  * alpha (float32, one value per (token, head, value channel)):
      "sigmoid_n21"    sigmoid(N(2, 1))
      "exp_softplus"   exp(-0.1 * softplus(N(0, 1)))
    With gate="scalar" alpha is one value per (token, head), and with
    gate="key" one per (token, head, key channel), same distributions, each
    drawn from its own tensor number; with gate="none" there is no alpha (None).
  * beta (float32, one scalar per (token, head)): sigmoid(N(0, 1)).
  * S0 (float32, [n_seq, H, d_v, d_k]): N(0, std^2) per element, or zeros.
  * Variable lengths: integers uniform on [lo, hi] inclusive from
    ``SeedSequence([seed, 1000])``, packed in draw order.

bf16 tensors are carried as numpy ``uint16`` bit patterns; ``bf16_to_f32``
widens them exactly.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_ELEMS = 1 << 22

# Tensor numbers inside a seed (fixed: changing them changes every workload).
_T_Q, _T_K, _T_V, _T_ALPHA, _T_BETA, _T_S0, _T_ALPHA_SCALAR, _T_ALPHA_KEY = 0, 1, 2, 3, 4, 5, 6, 7
_T_DO, _T_DST = 8, 9
GATES = ("channel", "scalar", "none", "key")


# ---------------------------------------------------------------- rounding ---
def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even); uint16 bits.

    Works on the float64 bit pattern directly (no double rounding through
    float32).  Meant for finite values in float32's normal range.
    """
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    b = (b + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    y = b.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of an input tensor as float32 (exact for both input dtypes)."""
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


# ------------------------------------------------------------------ draws ---
def _gen(seed: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, block])))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _blocked(n: int, fill, entry_elems: int):
    """Run fill(block_index, start, stop) over [0, n) in parallel threads."""
    block = max(1, BLOCK_ELEMS // max(1, entry_elems))
    starts = list(range(0, n, block))
    if len(starts) <= 1:
        for b, s in enumerate(starts):
            fill(b, s, min(n, s + block))
        return
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(lambda bs: fill(bs[0], bs[1], min(n, bs[1] + block)), enumerate(starts)))


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    return f64_to_bf16(x64) if dtype == "bf16" else x64.astype(np.float32)


def _empty(shape, dtype: str) -> np.ndarray:
    return np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)


def draw_unit_rows(seed, tensor, lead, d, dtype):
    """[*lead, d] array of N(0,1) rows, L2-normalised in float64, then rounded."""
    out = _empty((*lead, d), dtype)
    rest = int(np.prod(lead[1:], dtype=np.int64)) if len(lead) > 1 else 1

    def fill(b, s, e):
        x = _gen(seed, tensor, b).standard_normal((e - s, rest, d))
        x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        out.reshape(lead[0], rest, d)[s:e] = _round(x, dtype)

    _blocked(lead[0], fill, rest * d)
    return out


def draw_normal(seed, tensor, shape, dtype, std=1.0):
    out = _empty(shape, dtype)
    rest = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1

    def fill(b, s, e):
        x = _gen(seed, tensor, b).standard_normal((e - s, rest))
        if std != 1.0:
            x *= std
        out.reshape(shape[0], rest)[s:e] = _round(x, dtype)

    _blocked(shape[0], fill, rest)
    return out


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


ALPHA_KINDS = {
    "sigmoid_n21": lambda g, n: _sigmoid(g.standard_normal(n) + 2.0),
    "exp_softplus": lambda g, n: np.exp(-0.1 * _softplus(g.standard_normal(n))),
    # degenerate gates used by edge-case tests
    "ones": lambda g, n: np.ones(n),
    "zeros": lambda g, n: np.zeros(n),
}


def draw_mapped(seed, tensor, shape, fn):
    """float32 array of fn(generator, count) per block of the leading axis."""
    out = np.empty(shape, dtype=np.float32)
    rest = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1

    def fill(b, s, e):
        out.reshape(shape[0], rest)[s:e] = fn(_gen(seed, tensor, b), (e - s) * rest).reshape(e - s, rest)

    _blocked(shape[0], fill, rest)
    return out


def draw_lengths(seed: int, n_seq: int, lo: int, hi: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000])))
    return g.integers(lo, hi + 1, size=n_seq).astype(np.int64)


# --------------------------------------------------------------- packaging ---
@dataclass
class PrefillInputs:
    """Host arrays for one prefill call (token-major, packed sequences)."""
    q: np.ndarray            # [n_tok, H, d_k]  uint16 bf16 bits or float32
    k: np.ndarray            # [n_tok, H, d_k]
    v: np.ndarray            # [n_tok, H, d_v]
    alpha: Optional[np.ndarray]  # [n_tok, H, d_v] float32; [n_tok, H] (scalar gate); None (no gate)
    beta: np.ndarray         # [n_tok, H]       float32
    S0: Optional[np.ndarray]  # [n_seq, H, d_v, d_k] float32, or None (zeros)
    cu_seqlens: np.ndarray   # [n_seq+1] int64
    dtype: str               # "bf16" or "f32": dtype of q, k, v and o
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def n_tok(self):
        return int(self.q.shape[0])

    @property
    def n_seq(self):
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def H(self):
        return int(self.q.shape[1])

    @property
    def dk(self):
        return int(self.q.shape[2])

    @property
    def dv(self):
        return int(self.v.shape[2])

    def f32(self, name: str) -> np.ndarray:
        return as_f32(getattr(self, name), self.dtype)


@dataclass
class DecodeInputs:
    """Host arrays for n_steps successive decode steps (step-major)."""
    q: np.ndarray       # [n_steps, B, H, d_k]
    k: np.ndarray
    v: np.ndarray       # [n_steps, B, H, d_v]
    alpha: Optional[np.ndarray]  # [n_steps, B, H, d_v] float32; [n_steps, B, H] (scalar); None
    beta: np.ndarray    # [n_steps, B, H]      float32
    S0: np.ndarray      # [B, H, d_v, d_k]     float32
    dtype: str
    seed: int = 0
    meta: dict = field(default_factory=dict)

    def f32(self, name: str) -> np.ndarray:
        return as_f32(getattr(self, name), self.dtype)


def draw_gate(seed, lead, dv, alpha_kind, gate, dk=None):
    """alpha of shape [*lead, dv] (per value channel), [*lead, dk] (per key channel),
    [*lead] (scalar) or None (no gate)."""
    if gate == "channel":
        return draw_mapped(seed, _T_ALPHA, (*lead, dv), ALPHA_KINDS[alpha_kind])
    if gate == "scalar":
        return draw_mapped(seed, _T_ALPHA_SCALAR, tuple(lead), ALPHA_KINDS[alpha_kind])
    if gate == "key":
        return draw_mapped(seed, _T_ALPHA_KEY, (*lead, dk), ALPHA_KINDS[alpha_kind])
    if gate == "none":
        return None
    raise ValueError(f"gate must be one of {GATES}")


def make_prefill(seed: int, seq_lens, H: int, dk: int, dv: int, dtype: str = "bf16",
                 alpha_kind: str = "exp_softplus", s0_std: float = 0.0,
                 gate: str = "channel") -> PrefillInputs:
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    cu = np.zeros(len(seq_lens) + 1, dtype=np.int64)
    np.cumsum(seq_lens, out=cu[1:])
    n_tok = int(cu[-1])
    q = draw_unit_rows(seed, _T_Q, (n_tok, H), dk, dtype)
    k = draw_unit_rows(seed, _T_K, (n_tok, H), dk, dtype)
    v = draw_normal(seed, _T_V, (n_tok, H, dv), dtype)
    alpha = draw_gate(seed, (n_tok, H), dv, alpha_kind, gate, dk)
    beta = draw_mapped(seed, _T_BETA, (n_tok, H), lambda g, n: _sigmoid(g.standard_normal(n)))
    S0 = None
    if s0_std > 0.0:
        S0 = draw_normal(seed, _T_S0, (len(seq_lens), H, dv, dk), "f32", std=s0_std)
    return PrefillInputs(q, k, v, alpha, beta, S0, cu, dtype, seed,
                         dict(alpha_kind=alpha_kind, s0_std=s0_std, gate=gate))


def make_decode(seed: int, n_steps: int, B: int, H: int, dk: int, dv: int,
                dtype: str = "bf16", alpha_kind: str = "exp_softplus",
                s0_std: float = 0.02, gate: str = "channel") -> DecodeInputs:
    q = draw_unit_rows(seed, _T_Q, (n_steps, B, H), dk, dtype)
    k = draw_unit_rows(seed, _T_K, (n_steps, B, H), dk, dtype)
    v = draw_normal(seed, _T_V, (n_steps, B, H, dv), dtype)
    alpha = draw_gate(seed, (n_steps, B, H), dv, alpha_kind, gate, dk)
    beta = draw_mapped(seed, _T_BETA, (n_steps, B, H), lambda g, n: _sigmoid(g.standard_normal(n)))
    S0 = draw_normal(seed, _T_S0, (B, H, dv, dk), "f32", std=s0_std)
    return DecodeInputs(q, k, v, alpha, beta, S0, dtype, seed,
                        dict(alpha_kind=alpha_kind, s0_std=s0_std, gate=gate))


# The five workloads: shapes and distributions of the KDA prefill/decode path.
WORKLOADS = {
    1: dict(name="tiny_f32", kind="prefill", n_seq=1, T=256, H=1, dk=64, dv=64, dtype="f32",
            alpha_kind="sigmoid_n21", s0_std=0.0),
    2: dict(name="single_layer_prefill", kind="prefill", n_seq=1, T=4096, H=8, dk=128, dv=128,
            dtype="bf16", alpha_kind="exp_softplus", s0_std=0.0),
    3: dict(name="batched_prefill", kind="prefill", n_seq=4, T=8192, H=32, dk=128, dv=128,
            dtype="bf16", alpha_kind="exp_softplus", s0_std=0.02),
    4: dict(name="decode", kind="decode", B=256, steps=1024, H=32, dk=128, dv=128,
            dtype="bf16", alpha_kind="exp_softplus", s0_std=0.02),
    5: dict(name="varlen_prefill", kind="prefill", n_seq=64, len_lo=256, len_hi=16384, H=16,
            dk=128, dv=128, dtype="bf16", alpha_kind="exp_softplus", s0_std=0.0),
}


def workload_seed(wid: int) -> int:
    return 72000 + wid


def workload_seq_lens(wid: int) -> np.ndarray:
    w = WORKLOADS[wid]
    if "len_lo" in w:
        return draw_lengths(workload_seed(wid), w["n_seq"], w["len_lo"], w["len_hi"])
    return np.full(w["n_seq"], w["T"], dtype=np.int64)


def workload_prefill(wid: int, H: Optional[int] = None, seq_lens=None,
                     gate: str = "channel") -> PrefillInputs:
    """Inputs of a prefill workload; H / seq_lens may be overridden for reduced runs,
    and gate selects the layout of alpha (per channel, scalar, none)."""
    w = WORKLOADS[wid]
    assert w["kind"] == "prefill"
    lens = workload_seq_lens(wid) if seq_lens is None else np.asarray(seq_lens, dtype=np.int64)
    return make_prefill(workload_seed(wid), lens, H or w["H"], w["dk"], w["dv"], w["dtype"],
                        w["alpha_kind"], w["s0_std"], gate)


def workload_decode(wid: int = 4, n_steps: Optional[int] = None, B: Optional[int] = None,
                    H: Optional[int] = None, gate: str = "channel") -> DecodeInputs:
    w = WORKLOADS[wid]
    assert w["kind"] == "decode"
    return make_decode(workload_seed(wid), n_steps or w["steps"], B or w["B"], H or w["H"],
                       w["dk"], w["dv"], w["dtype"], w["alpha_kind"], w["s0_std"], gate)


def make_backward_grads(seed: int, inp: PrefillInputs):
    """Gradients flowing into a prefill call: dO [n_tok, H, d_v] and dS_T
    [n_seq, H, d_v, d_k], float32, standard normal."""
    n_tok, H, dv = inp.v.shape
    dk = inp.q.shape[2]
    dO = draw_normal(seed, _T_DO, (n_tok, H, dv), "f32")
    dS_T = draw_normal(seed, _T_DST, (inp.n_seq, H, dv, dk), "f32")
    return dO, dS_T
