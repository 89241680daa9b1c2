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
from tests import test_oracle_kda_pins as kda_pins
from tests import test_oracle_prefill_pins as prefill_pins
from tests import test_oracle_seam_pins as seam_pins

_SEAM_OUT = """  /* o_t = S_t^T q_t */
  const double *qt = sc->q + (((int64_t)b * c->N + t) * c->H + h) * dk;
  double *ot = sc->O + (((int64_t)b * c->N + t) * c->H + h) * dv;
  for (int j = 0; j < dv; ++j) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += qt[i] * S[i * dv + j];
    ot[j] = s;
  }
"""
_SEAM_UPDATE_START = "  if (sc->literal) {\n    token_transition(form, dk, kt, at, bt, Tt, NULL);"
_SEAM_LOOP = """    for (int64_t t = sc->seam_off[e]; t < sc->seam_off[e + 1]; ++t)
      seam_token(sc, b, h, t, S, Tt, tmp);
"""
_SEAM_PAIR_END = "    for (int i = 0; i < dk * dv; ++i) S[i] = tmp[i] + Sp[i];\n  }\n  free(Tt);"

_KDA_SEAM_GATE = """    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] *= at[i];
"""
_KDA_SEAM_READ = """    for (int j = 0; j < dv; ++j) {
      double s = 0.0;
      for (int i = 0; i < dk; ++i) s += kt[i] * S[i * dv + j];
      tmp[j] = s;
    }
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] += bt * kt[i] * (vt[j] - tmp[j]);
"""

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
    ("seam: output read before the token's update",
     [_SEAM_OUT, _SEAM_UPDATE_START],
     ["", _SEAM_OUT.replace("  const double *qt", "  {\n  const double *qt") + "  }\n"
      + _SEAM_UPDATE_START]),
    ("seam: window applied after the entry's pair",
     [_SEAM_LOOP, _SEAM_PAIR_END],
     ["", "    for (int i = 0; i < dk * dv; ++i) S[i] = tmp[i] + Sp[i];\n" + _SEAM_LOOP
      + "  }\n  free(Tt);"]),
    ("seam: output transposed",
     "for (int i = 0; i < dk; ++i) s += qt[i] * S[i * dv + j];",
     "for (int i = 0; i < dk; ++i) s += qt[i] * S[(j * dk + i) % (dk * dv)];"),
    ("seam: queries read with the value stride",
     "const double *qt = sc->q + (((int64_t)b * c->N + t) * c->H + h) * dk;",
     "const double *qt = sc->q + (((int64_t)b * c->N + t) * c->H + h) * dv;"),
    ("seam: first token of each window skipped",
     "for (int64_t t = sc->seam_off[e]; t < sc->seam_off[e + 1]; ++t)",
     "for (int64_t t = sc->seam_off[e] + (sc->seam_off[e + 1] > sc->seam_off[e]);"
     " t < sc->seam_off[e + 1]; ++t)"),
    ("seam: dense erase term dropped",
     "S[i * dv + j] = at[0] * (S[i * dv + j] - bt * kt[i] * tmp[j]) + bt * kt[i] * vt[j];",
     "S[i * dv + j] = at[0] * S[i * dv + j] + bt * kt[i] * vt[j];"),
    ("seam: diagonal gate of channel 0 for every row",
     "const double ai = (form == ORACLE_DIAG) ? at[i] : at[0];",
     "const double ai = at[0];"),
    ("KDA: gates applied after the erase (rows instead of columns)",
     "        t = e * at[j];",
     "        t = e * at[i];"),
    ("KDA: log scale of channel 0 instead of the largest gate",
     "      lam[0] += log(max_gate(at, dk));",
     "      lam[0] += log(at[0]);"),
    ("KDA specialised: ungated factor keeps the gate scale",
     "          Th[i * dk + j] *= at[i] / m;",
     "          Th[i * dk + j] *= at[i];"),
    ("KDA: smallest gate taken as the scale",
     "    if (at[i] > m) m = at[i];",
     "    if (at[i] < m) m = at[i];"),
    ("prefill: output read before the token's update",
     ["    if (c->O) {\n", "  for (int64_t t = t0; t < t1; ++t) {\n    const double *kt = k_at(c, b, t, h), *vt = v_at(c, b, t, h), *at = a_at(c, b, t, h);\n"],
     ["    if (0) {\n", "  for (int64_t t = t0; t < t1; ++t) {\n    if (c->O) {\n      const double *qt = c->q + (((int64_t)b * c->N + t) * c->H + h) * dk;\n      double *ot = c->O + (((int64_t)b * c->N + t) * c->H + h) * dv;\n      for (int j = 0; j < dv; ++j) {\n        double acc = 0.0;\n        for (int i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];\n        ot[j] = acc;\n      }\n    }\n    const double *kt = k_at(c, b, t, h), *vt = v_at(c, b, t, h), *at = a_at(c, b, t, h);\n"]),
    ("prefill: output transposed",
     "for (int i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];",
     "for (int i = 0; i < dk; ++i) acc += qt[i] * S[(j * dk + i) % (dk * dv)];"),
    ("prefill: queries read with the value stride",
     "const double *qt = c->q + (((int64_t)b * c->N + t) * c->H + h) * dk;",
     "const double *qt = c->q + (((int64_t)b * c->N + t) * c->H + h) * dv;"),
    ("prefill: output written to the previous token's row",
     "double *ot = c->O + (((int64_t)b * c->N + t) * c->H + h) * dv;",
     "double *ot = c->O + (((int64_t)b * c->N + (t > 0 ? t - 1 : 0)) * c->H + h) * dv;"),
    ("seam: KDA gates applied to the erase's key instead of the rows",
     "      for (int j = 0; j < dv; ++j) S[i * dv + j] *= at[i];\n    for (int j = 0; j < dv; ++j) {",
     "      for (int j = 0; j < dv; ++j) S[i * dv + j] *= 1.0;\n    for (int j = 0; j < dv; ++j) {"),
    ("seam: KDA erase read from the state before the gates",
     _KDA_SEAM_GATE + _KDA_SEAM_READ, _KDA_SEAM_READ + _KDA_SEAM_GATE),
    ("seam: KDA pair applied without its ungated operator",
     "        const double ungated = (form == ORACLE_DENSE || form == ORACLE_KDA)",
     "        const double ungated = (form == ORACLE_DENSE)"),
    ("seam: pair gate scale dropped",
     "Tp[i * dk + j] = exp(lp[nlam == 1 ? 0 : i]) * ungated;",
     "Tp[i * dk + j] = ungated;"),
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
    for form in (pins.SCALAR, pins.DIAG, pins.DENSE):
        calls += [
            lambda f=form: seam_pins.test_seam_split_equals_unsplit(f, False, [7, 9, 5], [0, 3, 3]),
            lambda f=form: seam_pins.test_seam_split_equals_unsplit(f, True, [4, 10, 3, 8],
                                                                    [0, 8, 8, 2]),
            lambda f=form: seam_pins.test_seam_exact_rational(f, 0),
            lambda f=form: seam_pins.test_seam_empty_windows_equal_compose(f),
            lambda f=form: seam_pins.test_seam_queries_only_reach_outputs(f),
        ]
    calls += [lambda: seam_pins.test_seam_split_equals_unsplit(oracle.KDA, False, [7, 9, 5],
                                                               [0, 3, 3]),
              lambda: seam_pins.test_seam_exact_rational(oracle.KDA, 0),
              seam_pins.test_seam_kda_with_shared_gates_is_the_dense_seam]
    calls.append(seam_pins.test_seam_delta_rule_retrieval)
    calls += [kda_pins.test_kda_literal_equals_specialised,
              lambda: kda_pins.test_kda_with_shared_gates_is_dense_gdn(False),
              lambda: kda_pins.test_kda_with_shared_gates_is_dense_gdn(True),
              kda_pins.test_kda_without_erase_is_diagonal,
              lambda: kda_pins.test_kda_exact_rational(0),
              lambda: kda_pins.test_kda_split_compose_equals_unsplit([0, 9, 10, 31]),
              kda_pins.test_kda_That_is_bounded]
    calls += [lambda: prefill_pins.test_plain_linear_attention_is_masked_product(False),
              prefill_pins.test_scalar_decay_closed_form,
              prefill_pins.test_diagonal_gate_closed_form,
              lambda: prefill_pins.test_outputs_are_prefix_recurrences_read_out(pins.DENSE),
              lambda: prefill_pins.test_delta_rule_retrieval(False)]
    for form in (pins.SCALAR, pins.DIAG, pins.DENSE):
        calls.append(lambda f=form: prefill_pins.test_exact_rational_brute_force(f, False))
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
    olds, news = (old, new) if isinstance(old, list) else ([old], [new])
    mutated = src
    for o, n in zip(olds, news):
        assert mutated.count(o) == 1, f"mutation target not found once: {name}"
        mutated = mutated.replace(o, n, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated, encoding="utf-8")
    so = str(tmp_path / "libmutant.so")
    oracle.compile_oracle(so, str(path))
    with np.errstate(all="ignore"):
        assert _caught(oracle.load(so)), f"no pin caught: {name}"
