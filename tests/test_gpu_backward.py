"""GPU parity of the prefill backward (kda_prefill_backward and its scalar-gate and key-gate forms)
against the fp64 backward oracle, through the C ABI.  The oracle side is pinned in
test_oracle_backward by central finite differences of the forward oracle."""
import numpy as np
import pytest

from gated_delta_rule_72_amd import inputs as I
from tests import helpers as Hh

pytestmark = pytest.mark.gpu

# fp32 arithmetic against fp64; gradients sum over up to d_v rows and many tokens
TOL = dict(max_rel=2e-4, rms_rel=1e-4)


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_72_amd import kda
    kda.lib()
    return torch


def run(torch, inp, gate, varlen, with_dST=True, want_dS0=True, seed=0):
    from gated_delta_rule_72_amd import kda
    from oracle.backward import prefill_backward
    dO, dS_T = I.make_backward_grads(9000 + seed, inp)
    if not with_dST:
        dS_T = None
    d = Hh.upload_prefill(inp)
    fn = {"channel": kda.kda_prefill_backward, "scalar": kda.kda_prefill_backward_scalar_gate,
          "none": kda.kda_prefill_backward_scalar_gate, "key": kda.kda_prefill_backward_key_gate}[gate]
    g = fn(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"] if varlen else None,
           Hh.to_device(dO, "f32"), None if dS_T is None else Hh.to_device(dS_T, "f32"), n_seq=inp.n_seq,
           want_dS0=want_dS0)
    torch.cuda.synchronize()
    ref = prefill_backward(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.alpha, inp.beta,
                           None if inp.S0 is None else inp.S0.astype(np.float64), inp.cu_seqlens, dO, dS_T, gate)
    H = inp.H
    sl = Hh.o_slices(inp.cu_seqlens, H)
    for name in ("dq", "dk", "dv", "dbeta"):
        Hh.check(name, Hh.from_device(g[name]), ref[name], sl, TOL)
    if gate != "none":
        Hh.check("dalpha", Hh.from_device(g["dalpha"]), ref["dalpha"], sl, TOL)
    if want_dS0:
        Hh.check("dS0", Hh.from_device(g["dS0"]), ref["dS0"], Hh.s_slices(inp.n_seq, H), TOL)
    else:
        assert g["dS0"] is None


@pytest.mark.parametrize("gate", ["channel", "scalar", "none", "key"])
@pytest.mark.parametrize("lens,H,dk,dv,dtype,varlen", [
    ([37, 1, 0, 20], 2, 64, 64, "f32", True),     # ragged blocks of 16, length 1, empty
    ([50], 3, 128, 128, "f32", False),
    ([33, 17], 2, 128, 64, "bf16", True),
    ([40, 25], 2, 64, 128, "f32", True),
    ([16, 16, 16], 1, 64, 64, "bf16", False),      # whole blocks only
])
def test_backward_matches_oracle(torch_cuda, gate, lens, H, dk, dv, dtype, varlen):
    print(f"backward gate={gate} lens={lens} H={H} dk={dk} dv={dv} {dtype} varlen={varlen}", flush=True)
    inp = I.make_prefill(9100 + sum(lens) + H + dk, lens, H, dk, dv, dtype, "exp_softplus", 0.02, gate)
    run(torch_cuda, inp, gate, varlen, seed=sum(lens))


def test_backward_without_state_gradients(torch_cuda):
    print("backward: no dS_T, no dS0, no S0", flush=True)
    inp = I.make_prefill(9201, [30, 45], 2, 128, 128, "f32", "sigmoid_n21", 0.0, "channel")
    run(torch_cuda, inp, "channel", True, with_dST=False, want_dS0=False, seed=1)


def test_backward_longer_sequences(torch_cuda):
    print("backward: 2 x 400 tokens, H=2, d=128, bf16", flush=True)
    inp = I.make_prefill(9202, [400, 400], 2, 128, 128, "bf16", "exp_softplus", 0.02, "channel")
    run(torch_cuda, inp, "channel", False, seed=2)


def test_backward_key_gate_longer_sequences(torch_cuda):
    print("backward, key-channel gate: 2 x 300 tokens, H=2, d=128, bf16", flush=True)
    inp = I.make_prefill(9203, [300, 300], 2, 128, 128, "bf16", "exp_softplus", 0.02, "key")
    run(torch_cuda, inp, "key", False, seed=3)


def test_backward_of_empty_sequences_passes_dS_T_through(torch_cuda):
    """Sequences with no tokens: S_T = S0, so dS0 = dS_T exactly, and the call writes
    nothing else (one non-empty sequence keeps the token tensors non-empty)."""
    print("backward: empty sequences", flush=True)
    from gated_delta_rule_72_amd import kda
    inp = I.make_prefill(9204, [0, 5, 0], 2, 64, 64, "f32", "exp_softplus", 0.02, "channel")
    dO, dS_T = I.make_backward_grads(9205, inp)
    d = Hh.upload_prefill(inp)
    g = kda.kda_prefill_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                                 Hh.to_device(dO, "f32"), Hh.to_device(dS_T, "f32"))
    torch_cuda.cuda.synchronize()
    dS0 = Hh.from_device(g["dS0"])
    np.testing.assert_array_equal(dS0[0], dS_T[0])
    np.testing.assert_array_equal(dS0[2], dS_T[2])
    run(torch_cuda, inp, "channel", True, seed=5)


# The forward pass that writes the state checkpoints takes 64 rows per workgroup when the
# call has a workgroup per CU or more (units x d_v / 64 >= 256), else 32 or 16 rows with 16
# lanes per row: 64 sequences x 4 heads at d_v = 128 select 64 rows, 32 x 2 select 32.
@pytest.mark.parametrize("n_seq,H,dtype,gate", [(64, 4, "f32", "channel"), (32, 2, "f32", "scalar"),
                                                (64, 4, "bf16", "key")])
def test_backward_checkpoint_variants(torch_cuda, n_seq, H, dtype, gate):
    lens = list(np.random.default_rng(n_seq + H).integers(20, 60, n_seq))
    print(f"backward gate={gate} {n_seq} sequences of 20-60 tokens, H={H}, d=128, {dtype}", flush=True)
    inp = I.make_prefill(9300 + n_seq + H, lens, H, 128, 128, dtype, "exp_softplus", 0.02, gate)
    run(torch_cuda, inp, gate, True, seed=n_seq + H)


# bf16 inputs with the value-channel, scalar or no gate take the chunked backward (64-token
# chunks on the matrix cores): ragged last chunks, a length-1 and an empty sequence, dense
# and packed calls, and all four (d_k, d_v) shapes.
@pytest.mark.parametrize("gate", ["channel", "scalar", "none"])
@pytest.mark.parametrize("lens,H,dk,dv,varlen", [
    ([200, 64, 1, 0, 130], 2, 128, 128, True),
    ([256], 2, 64, 128, False),
    ([300, 77], 3, 128, 64, True),
    ([129, 64], 2, 64, 64, True),
])
def test_chunked_backward_matches_oracle(torch_cuda, gate, lens, H, dk, dv, varlen):
    print(f"chunked backward gate={gate} lens={lens} H={H} dk={dk} dv={dv} varlen={varlen}", flush=True)
    inp = I.make_prefill(9400 + sum(lens) + H + dk + dv, lens, H, dk, dv, "bf16", "exp_softplus", 0.02, gate)
    run(torch_cuda, inp, gate, varlen, seed=sum(lens) + 7)


# Units the chunked form cannot take -- a chunk decaying past 2^-100 (here alpha = 0 on one
# token), a gate below 2^-5 (where dalpha = dg / alpha would amplify rounding), a beta of 0
# (dbeta divides by beta) -- are handed to the token-recurrent backward as whole (sequence,
# head) pairs, in the same call as the chunked units.
@pytest.mark.parametrize("gate", ["channel", "scalar"])
@pytest.mark.parametrize("kind", ["zero_gate", "small_gate", "zero_beta"])
def test_chunked_backward_hands_over_marked_units(torch_cuda, gate, kind):
    print(f"chunked backward, marked units: gate={gate} {kind}", flush=True)
    inp = I.make_prefill(9500 + len(kind), [150, 100], 3, 128, 128, "bf16", "exp_softplus", 0.02, gate)
    if kind == "zero_gate":
        inp.alpha[50, 1] = 0.0            # sequence 0, head 1
    elif kind == "small_gate":
        if gate == "channel":
            inp.alpha[170, 2, 7] = 0.01   # sequence 1, head 2, one value row
        else:
            inp.alpha[170, 2] = 0.01
    else:
        inp.beta[60, 0] = 0.0             # sequence 0, head 0
    run(torch_cuda, inp, gate, True, seed=len(kind) + 11)


def test_chunked_backward_batched_shape_sampled(torch_cuda):
    """The batched workload's shape on a reduced batch (2 x 8192 tokens, 4 heads, d = 128,
    bf16, its distributions): every gradient of two sampled (sequence, head) pairs against the
    oracle run on that pair alone (heads are independent)."""
    from gated_delta_rule_72_amd import kda
    from oracle.backward import prefill_backward
    inp = I.workload_prefill(3, H=4, seq_lens=[8192, 8192])
    print("chunked backward, 2 x 8192 tokens, H=4, d=128, bf16: sampled pairs", flush=True)
    dO, dS_T = I.make_backward_grads(9600, inp)
    d = Hh.upload_prefill(inp)
    g = kda.kda_prefill_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], None,
                                 Hh.to_device(dO, "f32"), Hh.to_device(dS_T, "f32"), n_seq=2)
    torch_cuda.cuda.synchronize()
    for n, h in [(0, 1), (1, 3)]:
        s, e = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        sub = lambda x: x[s:e, h:h + 1]
        ref = prefill_backward(sub(inp.f32("q")), sub(inp.f32("k")), sub(inp.f32("v")), sub(inp.alpha),
                               sub(inp.beta), inp.S0[n:n + 1, h:h + 1].astype(np.float64), [0, e - s], sub(dO),
                               dS_T[n:n + 1, h:h + 1], "channel")
        for name in ("dq", "dk", "dv", "dalpha", "dbeta"):
            Hh.check(f"{name}[{n},{h}]", Hh.from_device(g[name])[s:e, h], ref[name][:, 0], [(Ellipsis,)], TOL)
        Hh.check(f"dS0[{n},{h}]", Hh.from_device(g["dS0"])[n, h], ref["dS0"][0, 0], [(Ellipsis,)], TOL)
