"""GPU parity of the scalar-gate entry points (Gated DeltaNet: one forget gate per
(token, head) for every row; and the delta rule: no gate) against the fp64 oracle,
through the C ABI.  The oracle side is oracle.prefill_scalar_gate /
oracle.decode_scalar_gate, pinned in test_oracle_pins to a separately written
product-form loop of the scalar-gated delta rule."""
import numpy as np
import pytest

from gated_delta_rule_72_amd import inputs as I
from tests import helpers as Hh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_72_amd import kda
    kda.lib()
    return torch


def gpu_prefill(torch, inp, varlen=True):
    from gated_delta_rule_72_amd import kda
    d = Hh.upload_prefill(inp)
    o, S = kda.kda_prefill_scalar_gate(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                       d["cu_seqlens"] if varlen else None, n_seq=inp.n_seq)
    torch.cuda.synchronize()
    return Hh.from_device(o), Hh.from_device(S)


def oracle_prefill(inp, seqs=None, heads=None):
    """Oracle over whole sequences; seqs/heads restrict it to a subset (heads and
    sequences are independent, so a subset reproduces those outputs exactly)."""
    import oracle
    if seqs is None:
        return oracle.prefill_scalar_gate(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.alpha,
                                          inp.beta, None if inp.S0 is None else inp.S0.astype(np.float64),
                                          inp.cu_seqlens)
    out = {}
    for n in seqs:
        s, e = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        hs = list(heads)
        a = None if inp.alpha is None else inp.alpha[s:e][:, hs]
        S0 = None if inp.S0 is None else inp.S0[n:n + 1][:, hs].astype(np.float64)
        o, S = oracle.prefill_scalar_gate(inp.f32("q")[s:e][:, hs], inp.f32("k")[s:e][:, hs],
                                          inp.f32("v")[s:e][:, hs], a, inp.beta[s:e][:, hs], S0)
        for j, h in enumerate(hs):
            out[(n, h)] = (o[:, j], S[0, j])
    return out


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("lens,H,dk,dv,dtype,alpha_kind,s0", [
    ([256], 1, 64, 64, "f32", "sigmoid_n21", 0.0),
    ([200, 77, 1, 64], 2, 64, 64, "f32", "sigmoid_n21", 0.02),     # ragged tails, length 1
    ([130, 33], 2, 128, 128, "f32", "exp_softplus", 0.02),
    ([300, 64, 129], 4, 128, 128, "bf16", "exp_softplus", 0.02),
    ([513], 2, 64, 64, "bf16", "sigmoid_n21", 0.0),
    ([191, 2], 3, 128, 64, "bf16", "exp_softplus", 0.02),
    ([250], 2, 64, 128, "bf16", "exp_softplus", 0.02),
    ([0, 100, 0, 65], 2, 128, 128, "bf16", "exp_softplus", 0.02),  # empty sequences
])
def test_prefill_scalar_gate_matches_oracle(torch_cuda, gate, lens, H, dk, dv, dtype, alpha_kind, s0):
    print(f"prefill_scalar_gate gate={gate} lens={lens} H={H} dk={dk} dv={dv} {dtype} "
          f"{alpha_kind} s0={s0}", flush=True)
    inp = I.make_prefill(6100 + sum(lens) + H, lens, H, dk, dv, dtype, alpha_kind, s0, gate)
    o, S = gpu_prefill(torch_cuda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    tol = Hh.tol_for(dtype)
    Hh.check("o", o, o_ref, Hh.o_slices(inp.cu_seqlens, H), tol)
    Hh.check("S_T", S, S_ref, Hh.s_slices(inp.n_seq, H), tol)


def test_dense_call_and_unit_gate(torch_cuda):
    """Equal lengths without cu_seqlens give the varlen result bit for bit, and a scalar
    gate of all ones gives the no-gate result bit for bit (the same arithmetic)."""
    print("prefill_scalar_gate dense vs varlen, ones vs none", flush=True)
    inp = I.make_prefill(6200, [192, 192, 192], 2, 128, 128, "bf16", "exp_softplus", 0.02, "scalar")
    o1, S1 = gpu_prefill(torch_cuda, inp, varlen=True)
    o2, S2 = gpu_prefill(torch_cuda, inp, varlen=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)
    ones = I.make_prefill(6201, [130, 64], 2, 128, 128, "bf16", "ones", 0.02, "scalar")
    none = I.make_prefill(6201, [130, 64], 2, 128, 128, "bf16", "ones", 0.02, "none")
    oa, Sa = gpu_prefill(torch_cuda, ones)
    ob, Sb = gpu_prefill(torch_cuda, none)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(Sa, Sb)


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_batched_workload_scalar_gate_sampled(torch_cuda, gate):
    """The batched prefill workload's shapes (B=4 x 8192 tokens, H=32, d=128, bf16) with a
    scalar gate or none, as the benchmark launches it (dense, no cu_seqlens); oracle on
    sampled (sequence, head) pairs."""
    print(f"batched workload, gate={gate}: GPU whole problem, oracle on 3 pairs", flush=True)
    inp = I.workload_prefill(3, gate=gate)
    o, S = gpu_prefill(torch_cuda, inp, varlen=False)
    pairs = [(0, 0), (2, 17), (3, 31)]
    tol = Hh.tol_for(inp.dtype)
    for n, h in pairs:
        ref = oracle_prefill(inp, [n], [h])[(n, h)]
        s, e = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        Hh.check(f"o[seq={n},h={h}]", o[s:e, h], ref[0], [(Ellipsis,)], tol)
        Hh.check(f"S_T[seq={n},h={h}]", S[n, h], ref[1], [(Ellipsis,)], tol)


def run_decode(torch, dec):
    from gated_delta_rule_72_amd import kda
    dt = dec.dtype
    q, k, v = Hh.to_device(dec.q, dt), Hh.to_device(dec.k, dt), Hh.to_device(dec.v, dt)
    a = None if dec.alpha is None else Hh.to_device(dec.alpha, "f32")
    b = Hh.to_device(dec.beta, "f32")
    S = Hh.to_device(dec.S0, "f32").clone()
    outs = [kda.kda_decode_step_scalar_gate(q[t], k[t], v[t], None if a is None else a[t], b[t], S)
            for t in range(dec.q.shape[0])]
    torch.cuda.synchronize()
    return np.stack([Hh.from_device(x) for x in outs]), Hh.from_device(S)


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("B,H,dk,dv,dtype,steps", [
    (16, 4, 128, 128, "bf16", 48),
    (8, 3, 64, 64, "bf16", 40),
    (5, 2, 128, 64, "f32", 33),
    (3, 2, 64, 128, "f32", 17),
])
def test_decode_scalar_gate_matches_oracle(torch_cuda, gate, B, H, dk, dv, dtype, steps):
    import oracle
    print(f"decode_scalar_gate gate={gate} B={B} H={H} dk={dk} dv={dv} {dtype} steps={steps}",
          flush=True)
    dec = I.make_decode(6300 + B, steps, B, H, dk, dv, dtype, "exp_softplus", 0.02, gate)
    o, S = run_decode(torch_cuda, dec)
    o_ref, S_ref = oracle.decode_scalar_gate(dec.f32("q"), dec.f32("k"), dec.f32("v"), dec.alpha,
                                             dec.beta, dec.S0.astype(np.float64))
    tol = Hh.tol_for(dtype)
    Hh.check("o", o, o_ref, [(slice(None), b, h) for b in range(B) for h in range(H)], tol)
    Hh.check("S", S, S_ref, [(b, h) for b in range(B) for h in range(H)], tol)
