"""kda_prefill_noalloc (the prefill with the library's own device workspace) against
kda_prefill with a workspace of the caller, through the C ABI: the same kernels run, so
the outputs must agree bit for bit, and both must match the fp64 oracle at the bf16
tolerance.  Two calls in a row, the second on a smaller input: the array keeps the first
call's contents, which nothing may depend on."""
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


def test_noalloc_matches_prefill_on_two_calls(torch_cuda):
    from gated_delta_rule_72_amd import kda
    import oracle
    torch = torch_cuda
    # call 1: one 2048-token sequence, 2 heads (the sequence-parallel split: 16 segments, so the
    # workspace holds segment states too); call 2: three ragged sequences of 493 tokens in all,
    # 4 heads, fewer head-tokens than call 1 and a smaller workspace
    cases = [([2048], 2, False), ([300, 64, 129], 4, True)]
    for call, (lens, H, varlen) in enumerate(cases):
        print(f"noalloc call {call}: lens={lens} H={H} varlen={varlen}", flush=True)
        inp = I.make_prefill(8100 + call, lens, H, 128, 128, "bf16", "exp_softplus", 0.02)
        d = Hh.upload_prefill(inp)
        cu = d["cu_seqlens"] if varlen else None
        o1, S1 = kda.kda_prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], cu, n_seq=inp.n_seq)
        o2, S2 = kda.kda_prefill_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], cu,
                                         n_seq=inp.n_seq)
        torch.cuda.synchronize()
        o1, S1, o2, S2 = (Hh.from_device(x) for x in (o1, S1, o2, S2))
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
        o_ref, S_ref = oracle.prefill(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.alpha, inp.beta,
                                      inp.S0.astype(np.float64), inp.cu_seqlens)
        Hh.check("o", o2, o_ref, Hh.o_slices(inp.cu_seqlens, H), Hh.TOL_BF16)
        Hh.check("S_T", S2, S_ref, Hh.s_slices(inp.n_seq, H), Hh.TOL_BF16)


def test_noalloc_refuses_oversized_calls(torch_cuda):
    from gated_delta_rule_72_amd import kda
    # 16 sequences x 8192 tokens x 32 heads needs ~812 MB of solved A blocks: over the maximum
    L = kda.lib()
    need = kda.workspace_size(16, 16 * 8192, 32, 128, 128, kda.KDA_DTYPE_BF16)
    assert need > kda.NOALLOC_MAX_WORKSPACE
    A = 0x10000
    st = L.kda_prefill_noalloc(A, A, A, A, A, None, None, 16, 16 * 8192, 32, 128, 128, kda.KDA_DTYPE_BF16,
                               A, A, None)
    assert st == kda.KDA_ERR_WORKSPACE
