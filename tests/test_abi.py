"""C-ABI boundary checks that need no GPU: the library loads, exports every
symbol include/kda.h declares, and rejects bad arguments on the host before any
HIP call (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_72_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

A = 0x10000  # a 16-byte aligned fake device address; never dereferenced (rejected on host)


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    return kda.lib()


def test_every_declared_symbol_is_exported(L):
    syms = declared_symbols()
    assert set(syms) == set(kda.EXPORTED)
    for s in syms:
        assert hasattr(L, s), s


def test_version_and_status_strings(L):
    assert L.kda_abi_version() == 1
    for code, name in [(0, "KDA_OK"), (1, "KDA_ERR_INVALID_ARGUMENT"), (2, "KDA_ERR_UNSUPPORTED"),
                       (3, "KDA_ERR_DEVICE"), (4, "KDA_ERR_WORKSPACE")]:
        assert L.kda_status_string(code).decode() == name
    assert L.kda_status_string(99).decode() == "KDA_ERR_UNKNOWN"


def test_workspace_size(L):
    # fp32: the longest-first schedule (n_seq int32, 256-byte aligned)
    assert L.kda_prefill_workspace_size(64, 1000, 16, 128, 128, 0) == 256
    assert L.kda_prefill_workspace_size(65, 1000, 16, 128, 128, 0) == 512
    # bf16: schedule + chunk offsets (n_seq + 1 int32) + the decay-range marks (one int32
    # per (sequence, head, 64 value rows)) + one 12 KiB block of the solved
    # A = (I + L)^{-1} diag(beta) per (chunk, head), for at most n_tok // 64 + n_seq chunks
    rec = 3 * 2 * 32 * 32 * 2
    assert L.kda_prefill_workspace_size(64, 1000, 16, 128, 128, 1) == 256 + 512 + 8192 + (15 + 64) * 16 * rec
    assert L.kda_prefill_workspace_size(1, 0, 4, 64, 64, 1) == 256 + 256 + 256 + 1 * 4 * rec
    assert L.kda_prefill_workspace_size(0, 1000, 16, 128, 128, 1) == 0
    assert L.kda_prefill_workspace_size(4, 1000, 16, 96, 128, 1) == 0


def test_key_gate_workspace_size(L):
    """The key-channel-gate prefill: fp32 as kda_prefill; bf16: schedule, chunk offsets,
    one flag per (sequence, head, 64 value rows), one mark per (chunk, head), then two
    12 KiB solved records per (chunk, head) -- A and the decayed Q K^T -- for at most
    n_tok // 64 + n_seq chunks; every part 256-byte aligned, never split into segments."""
    al = lambda x: (x + 255) // 256 * 256
    rec = 3 * 2 * 32 * 32 * 2

    def size(n_seq, n_tok, H, dv):
        mc = n_tok // 64 + n_seq
        return (al(n_seq * 4) + al((n_seq + 1) * 4) + al(n_seq * H * (dv // 64) * 4) + al(mc * H * 4)
                + 2 * al(mc * H * rec))

    assert L.kda_prefill_key_gate_workspace_size(64, 1000, 16, 128, 128, 0) == 256
    assert L.kda_prefill_key_gate_workspace_size(64, 1000, 16, 128, 128, 1) == size(64, 1000, 16, 128)
    assert L.kda_prefill_key_gate_workspace_size(1, 4096, 8, 128, 128, 1) == size(1, 4096, 8, 128)
    assert L.kda_prefill_key_gate_workspace_size(4, 32768, 32, 128, 128, 1) == size(4, 32768, 32, 128)
    assert L.kda_prefill_key_gate_workspace_size(3, 500, 2, 64, 128, 1) == size(3, 500, 2, 128)
    assert L.kda_prefill_key_gate_workspace_size(0, 1000, 16, 128, 128, 1) == 0
    assert L.kda_prefill_key_gate_workspace_size(4, 1000, 16, 96, 128, 1) == 0


def test_workspace_size_of_split_calls(L):
    """Calls with few (sequence, head) units are split into G segments per sequence
    (G >= 4, units x G <= 256, on average two chunks or more per segment); their
    workspace adds the segment bookkeeping and states.  Layout, 256-byte aligned parts:
    order NS int32, chunk offsets NS+1, segment offsets NS+1 (split calls only),
    decay-range marks NS x H x d/64 int32, A records (n_tok/64 + n_seq) x H x 12 KiB,
    then dS, M, S_start (NS x H x d x d fp32 each) and the total decays (NS x H x d fp32),
    NS = n_seq G."""
    al = lambda x: (x + 255) // 256 * 256
    rec = 3 * 2 * 32 * 32 * 2

    def split_size(n_seq, n_tok, H, d, G):
        ns = n_seq * G
        return (al(ns * 4) + al((ns + 1) * 4) + al((ns + 1) * 4) + al(ns * H * (d // 64) * 4)
                + al((n_tok // 64 + n_seq) * H * rec) + 3 * ns * H * d * d * 4 + al(ns * H * d * 4))

    # one 4096-token sequence, 8 heads, d = 128: 16 units -> G = 16
    assert L.kda_prefill_workspace_size(1, 4096, 8, 128, 128, 1) == split_size(1, 4096, 8, 128, 16)
    # 65,573 tokens, 4 heads: 8 units -> G = 32
    assert L.kda_prefill_workspace_size(1, 65573, 4, 128, 128, 1) == split_size(1, 65573, 4, 128, 32)
    # d = 64, one head: 1 unit, 2048 tokens -> G = 16
    assert L.kda_prefill_workspace_size(1, 2048, 1, 64, 64, 1) == split_size(1, 2048, 1, 64, 16)
    # 512 tokens, 8 heads: 16 units, segments of two chunks -> G = 4
    assert L.kda_prefill_workspace_size(1, 512, 8, 128, 128, 1) == split_size(1, 512, 8, 128, 4)
    # not split: 256 units (the batched workload), G < 4 (two sequences of 8192 tokens,
    # 32 heads: G would be 2), segments too short (256 tokens, 8 heads: G would be 2),
    # d_k != d_v, fp32
    unsplit = lambda n_seq, n_tok, H, dv=128: (al(n_seq * 4) + al((n_seq + 1) * 4) + al(n_seq * H * (dv // 64) * 4)
                                               + al((n_tok // 64 + n_seq) * H * rec))
    assert L.kda_prefill_workspace_size(4, 32768, 32, 128, 128, 1) == unsplit(4, 32768, 32)
    assert L.kda_prefill_workspace_size(2, 16384, 32, 128, 128, 1) == unsplit(2, 16384, 32)
    assert L.kda_prefill_workspace_size(1, 256, 8, 128, 128, 1) == unsplit(1, 256, 8)
    assert L.kda_prefill_workspace_size(1, 1024, 8, 128, 128, 1) == split_size(1, 1024, 8, 128, 8)
    assert L.kda_prefill_workspace_size(1, 4096, 8, 128, 64, 1) == unsplit(1, 4096, 8, 64)
    assert L.kda_prefill_workspace_size(1, 4096, 8, 128, 128, 0) == 256


def prefill(L, fn="kda_prefill", **kw):
    args = dict(q=A, k=A + 0x100000, v=A + 0x200000, alpha=A + 0x300000, beta=A + 0x400000,
                S0=None, cu=None, n_seq=2, n_tok=64, H=2, dk=64, dv=64, dt=1,
                o=A + 0x500000, S_T=A + 0x600000, ws=A + 0x700000, ws_bytes=256, stream=None)
    args.update(kw)
    return getattr(L, fn)(args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["S0"],
                         args["cu"], args["n_seq"], args["n_tok"], args["H"], args["dk"], args["dv"],
                         args["dt"], args["o"], args["S_T"], args["ws"], args["ws_bytes"],
                         args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(n_seq=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(n_tok=-1), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(H=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(n_tok=63), kda.KDA_ERR_INVALID_ARGUMENT),          # not a multiple of n_seq, no cu_seqlens
    (dict(q=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(o=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(beta=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(k=A + 0x100008), kda.KDA_ERR_INVALID_ARGUMENT),   # misaligned
    (dict(S_T=A + 0x600004), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(o=A), kda.KDA_ERR_INVALID_ARGUMENT),              # o overlaps q
    (dict(S0=A + 0x600000 + 16, S_T=A + 0x600000), kda.KDA_ERR_INVALID_ARGUMENT),  # partial overlap
    (dict(ws=None), kda.KDA_ERR_WORKSPACE),
    (dict(ws_bytes=128), kda.KDA_ERR_WORKSPACE),
    (dict(ws=A + 0x500000, ws_bytes=1 << 20), kda.KDA_ERR_INVALID_ARGUMENT),  # workspace overlaps o
])
def test_prefill_rejects_on_host(L, kw, status):
    assert prefill(L, **kw) == status


def decode(L, fn="kda_decode_step", **kw):
    args = dict(q=A, k=A + 0x100000, v=A + 0x200000, alpha=A + 0x300000, beta=A + 0x400000,
                S=A + 0x1000000, o=A + 0x500000, B=4, H=2, dk=128, dv=128, dt=1, stream=None)
    args.update(kw)
    return getattr(L, fn)(args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["S"],
                             args["o"], args["B"], args["H"], args["dk"], args["dv"], args["dt"],
                             args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(B=-1), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(H=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dk=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(S=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(alpha=A + 0x300002), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(beta=A + 0x400002), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(S=A), kda.KDA_ERR_INVALID_ARGUMENT),              # S overlaps q
    (dict(o=A + 0x1000000 + 64), kda.KDA_ERR_INVALID_ARGUMENT),  # o inside S
    (dict(B=0), kda.KDA_OK),                                # nothing to do, nothing enqueued
])
def test_decode_rejects_on_host(L, kw, status):
    assert decode(L, **kw) == status


# Scalar-gate entry points: alpha is [n_tok, H] (4-byte aligned) or NULL (no gate).
# Only rejections are exercised here: an accepted call would reach the device.
@pytest.mark.parametrize("kw,status", [
    (dict(alpha=A + 0x300002), kda.KDA_ERR_INVALID_ARGUMENT),   # not 4-byte aligned
    (dict(alpha=None, beta=None), kda.KDA_ERR_INVALID_ARGUMENT),  # no gate is fine, no beta is not
    (dict(alpha=None, o=A), kda.KDA_ERR_INVALID_ARGUMENT),     # o overlaps q
    (dict(alpha=None, dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(alpha=None, ws=None), kda.KDA_ERR_WORKSPACE),
    # the scalar gate spans n_tok * H * 4 = 512 bytes: o placed inside it overlaps
    (dict(o=A + 0x300000 + 256), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(alpha=A + 0x500000 - 512 + 4), kda.KDA_ERR_INVALID_ARGUMENT),  # its tail overlaps o
])
def test_prefill_scalar_gate_rejects_on_host(L, kw, status):
    assert prefill(L, "kda_prefill_scalar_gate", **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(alpha=A + 0x300002), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(alpha=None, S=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(alpha=None, S=A), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(alpha=A + 0x1000000), kda.KDA_ERR_INVALID_ARGUMENT),  # the gate inside S
    (dict(alpha=None, B=0), kda.KDA_OK),
])
def test_decode_scalar_gate_rejects_on_host(L, kw, status):
    assert decode(L, "kda_decode_step_scalar_gate", **kw) == status


def test_binding_refuses_cpu_tensors(L):
    torch = pytest.importorskip("torch")
    q = torch.zeros(4, 2, 64)
    with pytest.raises(ValueError, match="GPU tensors only"):
        kda.kda_decode_step(q, q, q, q, torch.zeros(4, 2), torch.zeros(4, 2, 64, 64))


def _prefill_args(torch, n_tok=32, H=2, dk=64, dv=128, n_seq=2, dt=None):
    dt = dt or torch.bfloat16
    f = torch.float32
    return dict(q=torch.zeros(n_tok, H, dk, dtype=dt), k=torch.zeros(n_tok, H, dk, dtype=dt),
                v=torch.zeros(n_tok, H, dv, dtype=dt), alpha=torch.zeros(n_tok, H, dv, dtype=f),
                beta=torch.zeros(n_tok, H, dtype=f), S0=torch.zeros(n_seq, H, dv, dk, dtype=f))


@pytest.mark.parametrize("change,match", [
    (lambda t, a: a.update(k=a["k"].float()), "k must be"),                     # k not q's dtype
    (lambda t, a: a.update(v=a["v"][:, :1].contiguous()), "v must be"),          # v of other heads
    (lambda t, a: a.update(alpha=a["alpha"][..., :64].contiguous()), "alpha must have shape"),  # key-gate shape
    (lambda t, a: a.update(alpha=a["alpha"].double()), "alpha must be"),
    (lambda t, a: a.update(alpha=None), "alpha is required"),
    (lambda t, a: a.update(beta=a["beta"].to(t.bfloat16)), "beta must be"),
    (lambda t, a: a.update(S0=a["S0"][:1].contiguous()), "S0 must have shape"),
    (lambda t, a: a.update(S0=a["S0"].transpose(2, 3).contiguous()), "S0 must have shape"),
])
def test_binding_checks_prefill_shapes_and_dtypes(L, change, match):
    """The binding rejects mismatched tensors with ValueError before any library call
    (the C ABI sees raw pointers only); CPU tensors suffice, nothing reaches the device."""
    torch = pytest.importorskip("torch")
    a = _prefill_args(torch)
    change(torch, a)
    with pytest.raises(ValueError, match=match):
        kda.kda_prefill(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, n_seq=2)


def test_binding_checks_gate_forms(L):
    torch = pytest.importorskip("torch")
    a = _prefill_args(torch)
    # the scalar gate takes [n_tok, H] (or None); the key-channel gate [n_tok, H, d_k]
    with pytest.raises(ValueError, match=r"alpha must have shape \(32, 2\)"):
        kda.kda_prefill_scalar_gate(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, n_seq=2)
    with pytest.raises(ValueError, match=r"alpha must have shape \(32, 2, 64\)"):
        kda.kda_prefill_key_gate(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, n_seq=2)
    # no gate passes the checks and is refused only for being on the CPU
    with pytest.raises(ValueError, match="GPU tensors only"):
        kda.kda_prefill_scalar_gate(a["q"], a["k"], a["v"], None, a["beta"], a["S0"], None, n_seq=2)
    with pytest.raises(ValueError, match="o must be"):
        kda.kda_prefill(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, n_seq=2,
                        o=torch.zeros(32, 2, 128))
    with pytest.raises(ValueError, match="S_T must have shape"):
        kda.kda_prefill(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, n_seq=2,
                        S_T=torch.zeros(2, 2, 64, 128))


def test_binding_checks_backward_gradients(L):
    """A bf16 call's o is bf16; the backward takes dO in float32 and says so, instead of
    reading a half-size buffer as float32."""
    torch = pytest.importorskip("torch")
    a = _prefill_args(torch)
    dO_bf16 = torch.zeros(32, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dO must be"):
        kda.kda_prefill_backward(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, dO_bf16, n_seq=2)
    dO = torch.zeros(32, 2, 128)
    with pytest.raises(ValueError, match="dS_T must have shape"):
        kda.kda_prefill_backward(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, dO,
                                 torch.zeros(2, 2, 128, 128), n_seq=2)
    with pytest.raises(ValueError, match="alpha must have shape"):
        kda.kda_prefill_backward_scalar_gate(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], None, dO,
                                             n_seq=2)
    with pytest.raises(ValueError, match="k must be"):
        kda.kda_prefill_backward(a["q"], a["k"].float(), a["v"], a["alpha"], a["beta"], a["S0"], None, dO, n_seq=2)


def test_binding_checks_decode_shapes(L):
    torch = pytest.importorskip("torch")
    bf = torch.bfloat16
    q = torch.zeros(4, 2, 64, dtype=bf)
    v = torch.zeros(4, 2, 128, dtype=bf)
    S = torch.zeros(4, 2, 128, 64)
    with pytest.raises(ValueError, match="alpha must have shape"):
        kda.kda_decode_step(q, q, v, torch.zeros(4, 2, 64), torch.zeros(4, 2), S)
    with pytest.raises(ValueError, match="S must have shape"):
        kda.kda_decode_step(q, q, v, torch.zeros(4, 2, 128), torch.zeros(4, 2), torch.zeros(4, 2, 64, 128))
    with pytest.raises(ValueError, match="beta must be"):
        kda.kda_decode_step_scalar_gate(q, q, v, None, torch.zeros(4, 2, dtype=torch.float64), S)


def test_backward_workspace_size(L):
    """Backward workspace, 256-byte aligned parts: the schedule (n_seq int32), the chunk
    offsets (n_seq + 1 int32) and the unit marks (n_seq x H x d_v / 64 int32), then one region
    that is the larger of the chunked path's -- a 12 KiB solved record, the entering state and
    the leaving-state gradient (d_v x d_k fp32 each) per (chunk, head), for n_tok // 64 + n_seq
    chunks -- and the token-recurrent path's: a state checkpoint every 16 tokens of every
    (sequence, head) (slots n_seq + n_tok // 16 + 1, H x d_v x d_k fp32 each) and each wave's
    16 states of 8 rows (d_k fp32 each; one wave per 8 value rows, (sequence, head) pairs padded
    to a multiple of 8)."""
    al = lambda x: (x + 255) // 256 * 256

    def size(n_seq, n_tok, H, dk, dv):
        prefix = al(n_seq * 4) + al((n_seq + 1) * 4) + al(n_seq * H * (dv // 64) * 4)
        mc = n_tok // 64 + n_seq
        chunked = al(mc * H * 12288) + 2 * al(mc * H * dv * dk * 4)
        waves = (n_seq * H + 7) // 8 * 8 * (dv // 8)
        recurrent = al(al((n_seq + n_tok // 16 + 1) * H * dv * dk * 4) + waves * 16 * 8 * dk * 4)
        return prefix + max(chunked, recurrent)

    for shape in [(1, 256, 1, 64, 64), (4, 1000, 3, 128, 64), (3, 0, 2, 64, 128), (65, 4096, 8, 128, 128)]:
        assert L.kda_prefill_backward_workspace_size(*shape) == size(*shape)
    assert L.kda_prefill_backward_workspace_size(0, 16, 1, 64, 64) == 0
    assert L.kda_prefill_backward_workspace_size(1, 16, 1, 96, 64) == 0


def backward(L, fn="kda_prefill_backward", **kw):
    M = 0x100000
    args = dict(q=A, k=A + M, v=A + 2 * M, alpha=A + 3 * M, beta=A + 4 * M, S0=None, cu=None,
                dO=A + 5 * M, dS_T=None, n_seq=2, n_tok=64, H=2, dk=64, dv=64, dt=1,
                dq=A + 6 * M, dk_=A + 7 * M, dv_=A + 8 * M, dalpha=A + 9 * M, dbeta=A + 10 * M,
                dS0=A + 11 * M, ws=A + 32 * M, ws_bytes=1 << 24, stream=None)
    args.update(kw)
    a = args
    return getattr(L, fn)(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"], a["cu"], a["dO"], a["dS_T"],
                          a["n_seq"], a["n_tok"], a["H"], a["dk"], a["dv"], a["dt"], a["dq"], a["dk_"], a["dv_"],
                          a["dalpha"], a["dbeta"], a["dS0"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("fn", ["kda_prefill_backward", "kda_prefill_backward_scalar_gate",
                                "kda_prefill_backward_key_gate"])
@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(n_seq=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(n_tok=63), kda.KDA_ERR_INVALID_ARGUMENT),          # not a multiple of n_seq, no cu_seqlens
    (dict(dO=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dq=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dbeta=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dq=A + 6 * 0x100000 + 8), kda.KDA_ERR_INVALID_ARGUMENT),   # misaligned
    (dict(dv_=A + 8 * 0x100000 + 2), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dq=A + 0x100), kda.KDA_ERR_INVALID_ARGUMENT),               # dq overlaps q
    (dict(dk_=A + 6 * 0x100000 + 0x100), kda.KDA_ERR_INVALID_ARGUMENT),  # dk overlaps dq
    (dict(ws=None), kda.KDA_ERR_WORKSPACE),
    (dict(ws_bytes=4096), kda.KDA_ERR_WORKSPACE),
    (dict(ws=A + 11 * 0x100000), kda.KDA_ERR_INVALID_ARGUMENT),       # workspace overlaps dS0
])
def test_backward_rejects_on_host(L, fn, kw, status):
    assert backward(L, fn, **kw) == status


def test_backward_gate_needs_its_gradient(L):
    assert backward(L, dalpha=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert backward(L, alpha=None) == kda.KDA_ERR_INVALID_ARGUMENT


def test_backward_key_gate_needs_aligned_alpha(L):
    fn = "kda_prefill_backward_key_gate"
    assert backward(L, fn, alpha=A + 3 * 0x100000 + 4) == kda.KDA_ERR_INVALID_ARGUMENT
    # a scalar gate is read as scalars: 4-byte alignment, so 2 bytes off is rejected
    assert backward(L, "kda_prefill_backward_scalar_gate", alpha=A + 3 * 0x100000 + 2) == kda.KDA_ERR_INVALID_ARGUMENT


def test_noalloc_refuses_oversized_calls_on_host(L):
    """kda_prefill_noalloc checks the workspace its sizes need against the array it holds
    (KDA_PREFILL_NOALLOC_MAX_WORKSPACE) with host arithmetic alone, before any HIP call."""
    assert kda.NOALLOC_MAX_WORKSPACE == 256 << 20
    n_tok = 16 * 8192
    assert L.kda_prefill_workspace_size(16, n_tok, 32, 128, 128, 1) > kda.NOALLOC_MAX_WORKSPACE
    st = L.kda_prefill_noalloc(A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, None, None, 16, n_tok,
                               32, 128, 128, 1, A + 0x500000, A + 0x600000, None)
    assert st == kda.KDA_ERR_WORKSPACE
