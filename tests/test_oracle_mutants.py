"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake (a dropped term, a wrong sign, a wrong index, a
transposed operand, a reversed product) in a temporary copy of the oracle's C
source, builds it on the CPU, and checks that at least one pin of
``test_oracle_pins`` fails against it.  The real oracle is never modified.
"""

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = [
    ("dense: gate dropped from the state update",
     "S[i * dv + j] = a * (S[i * dv + j] - bt * kt[i] * kS[j]) + bt * kt[i] * vt[j];",
     "S[i * dv + j] = (S[i * dv + j] - bt * kt[i] * kS[j]) + bt * kt[i] * vt[j];"),
    ("dense: erase term with the wrong sign",
     "S[i * dv + j] = a * (S[i * dv + j] - bt * kt[i] * kS[j]) + bt * kt[i] * vt[j];",
     "S[i * dv + j] = a * (S[i * dv + j] + bt * kt[i] * kS[j]) + bt * kt[i] * vt[j];"),
    ("dense: beta dropped from the write term",
     "S[i * dv + j] = a * (S[i * dv + j] - bt * kt[i] * kS[j]) + bt * kt[i] * vt[j];",
     "S[i * dv + j] = a * (S[i * dv + j] - bt * kt[i] * kS[j]) + kt[i] * vt[j];"),
    ("dense: ungated factor misses beta",
     "Th[i * dk + j] -= bt * kt[i] * kS[j];",
     "Th[i * dk + j] -= kt[i] * kS[j];"),
    ("diag: gate index fixed to channel 0",
     "S[i * dv + j] = at[i] * S[i * dv + j] + kt[i] * vt[j];",
     "S[i * dv + j] = at[0] * S[i * dv + j] + kt[i] * vt[j];"),
    ("diag: log gate of channel 0 for every channel",
     "for (int i = 0; i < nlam; ++i) lam[i] += log(at[i]);",
     "for (int i = 0; i < nlam; ++i) lam[i] += log(at[0]);"),
    ("scalar: operator not decayed",
     "for (int i = 0; i < dk * dk; ++i) T[i] *= a;",
     "for (int i = 0; i < dk * dk; ++i) T[i] *= 1.0;"),
    ("literal: product order reversed (earliest on the left)",
     "matmul(dk, dk, dk, Tt, T, tmpT);",
     "matmul(dk, dk, dk, T, Tt, tmpT);"),
    ("literal: state not carried through the token transition",
     "      matmul(dk, dk, dv, Tt, S, tmpS);",
     "      memcpy(tmpS, S, sizeof(double) * dk * dv);"),
    ("build: first token of each segment skipped",
     "for (int64_t t = t0; t < t1; ++t) {",
     "for (int64_t t = t0 + (t1 > t0 ? 1 : 0); t < t1; ++t) {"),
    ("compose: operator transposed",
     "T[i * dk + j] = scale * th;",
     "T[j * dk + i] = scale * th;"),
    ("compose: gate scale dropped",
     "double scale = exp(lp[form == ORACLE_DIAG ? i : 0]);",
     "double scale = 1.0;"),
    ("compose: chain operator multiplied in the wrong order",
     "matmul(dk, dk, dk, c->That + unit * dk * dk, Tacc, Ttmp);",
     "matmul(dk, dk, dk, Tacc, c->That + unit * dk * dk, Ttmp);"),
    ("compose: S(C|0) added before the operator is applied",
     "    matmul(dk, dk, dv, T, S, tmp);\n    for (int i = 0; i < dk * dv; ++i) S[i] = tmp[i] + Sp[i];",
     "    for (int i = 0; i < dk * dv; ++i) S[i] += Sp[i];\n    matmul(dk, dk, dv, T, S, tmp);\n    for (int i = 0; i < dk * dv; ++i) S[i] = tmp[i];"),
    ("value rows read with the key stride",
     "return c->v + (((int64_t)b * c->N + t) * c->H + h) * c->dv;",
     "return c->v + (((int64_t)b * c->N + t) * c->H + h) * c->dk;"),
]


def _pin_calls():
    """Every pin, as zero-argument callables (a representative parameter set)."""
    calls = []
    for ex in pins.HAND:
        for lit in (False, True):
            calls.append(lambda ex=ex, lit=lit: pins.test_hand_examples(ex, lit))
    for form in (pins.SCALAR, pins.DIAG, pins.DENSE):
        calls += [
            lambda f=form: pins.test_p1_split_compose_equals_unsplit(f, [0, 1, 40, 41, 90]),
            lambda f=form: pins.test_literal_equals_specialised(f),
            lambda f=form: pins.test_p6_associativity(f),
            lambda f=form: pins.test_p7_naive_error(f),
            lambda f=form: pins.test_p10_exact_rational_brute_force(f, 0),
        ]
    calls += [pins.test_p3_vanilla_linear_attention, pins.test_p4_scalar_closed_form,
              pins.test_p5_diag_closed_form, pins.test_p9_delta_rule_retrieval,
              pins.test_p11_one_hot_closed_form, pins.test_p12_permutation_chain,
              lambda: pins.test_p2_identity_dense(False)]
    return calls


def _caught(lib):
    saved = oracle.load
    oracle.load = lambda path=None: lib
    try:
        for call in _pin_calls():
            try:
                call()
            except (AssertionError, ValueError, FloatingPointError):
                return True
    finally:
        oracle.load = saved
    return False


def test_real_oracle_passes_every_pin():
    assert not _caught(oracle.load())


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(oracle._SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation target not found: {name}"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated, encoding="utf-8")
    so = str(tmp_path / "libmutant.so")
    oracle.compile_oracle(so, str(path))
    with np.errstate(all="ignore"):
        assert _caught(oracle.load(so)), f"no pin caught: {name}"
