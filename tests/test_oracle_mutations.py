"""The oracle pins must catch plausible slips: each mutant of the oracle's C
source (a dropped term, a wrong sign or index, a transposed operand, the
read-out taken before the update) is compiled on the CPU and must fail at least
one pin.  The real oracle is restored afterwards."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, exact text in kda_oracle.c, replacement)
MUTANTS = [
    ("decay_on_key_columns", "for (int64_t j = 0; j < dk; ++j) Si[j] *= ai;",
     "for (int64_t j = 0; j < dk; ++j) Si[j] *= (double)at[j % dv];"),
    ("no_forget_gate", "for (int64_t j = 0; j < dk; ++j) Si[j] *= ai;", "(void)ai;"),
    ("error_sign_flipped", "e[i] = bt * ((double)vt[i] - vp[i]);", "e[i] = bt * ((double)vt[i] + vp[i]);"),
    ("beta_dropped", "e[i] = bt * ((double)vt[i] - vp[i]);", "e[i] = ((double)vt[i] - vp[i]) + 0.0 * bt;"),
    ("beta_of_previous_token", "const double bt = (double)beta[t * b_stride];",
     "const double bt = (double)beta[(t > 0 ? t - 1 : 0) * b_stride];"),
    ("readout_before_update", "for (int64_t j = 0; j < dk; ++j) acc += Si[j] * (double)qt[j];",
     "for (int64_t j = 0; j < dk; ++j) acc += (Si[j] - e[i] * (double)kt[j]) * (double)qt[j];"),
    ("predict_with_query", "for (int64_t j = 0; j < dk; ++j) acc += Si[j] * (double)kt[j];",
     "for (int64_t j = 0; j < dk; ++j) acc += Si[j] * (double)qt[j];"),
    ("update_with_query", "for (int64_t j = 0; j < dk; ++j) Si[j] += ei * (double)kt[j];",
     "for (int64_t j = 0; j < dk; ++j) Si[j] += ei * (double)qt[j];"),
]

PIN_TESTS = [
    pins.test_hand_worked_example_d2_t2,
    pins.test_T1_closed_form_any_S0,
    pins.test_T2_hand_expanded_zero_start,
    pins.test_T3_unrolled_rank_one_sum,
    pins.test_alpha_zero_forgets_everything,
    pins.test_orthonormal_keys_are_stored_exactly_and_give_linear_attention,
    pins.test_beta_zero_is_pure_decay,
    pins.test_householder_reflections_preserve_frobenius_norm,
]


def _build_mutant(src_text, tmpdir, name):
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as fh:
        fh.write(src_text)
    lib = os.path.join(tmpdir, f"lib{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", path, "-o", lib],
                   check=True)
    return lib


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught_by_a_pin(name, old, new, monkeypatch):
    text = open(SRC).read()
    assert old in text, f"mutation anchor for {name} not found"
    tmpdir = tempfile.mkdtemp(prefix="kda_mutant_")
    try:
        lib = _build_mutant(text.replace(old, new, 1), tmpdir, name)
        monkeypatch.setattr(oracle, "_LIB_PATH", lib)
        monkeypatch.setattr(oracle, "_lib", None)
        failures = 0
        for pin in PIN_TESTS:
            try:
                pin()
            except AssertionError:
                failures += 1
        assert failures > 0, f"no pin caught mutant {name}"
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    monkeypatch.setattr(oracle, "_lib", None)
