"""Pins of the oracle's prefill with per-token outputs (``oracle.prefill``).

A segment prefilled on its own gives, besides its pair, every token's output
o_t = S_t^T q_t read from the state right after the token's update.  The
pins fix it against what does not come from the prefill code itself:

* plain causal linear attention (scalar form, alpha = 1): O = tril(Q K^T) V
  per segment, a numpy matrix product;
* decayed and gated causal attention in closed form (scalar and diagonal
  forms: suffix products of the gates);
* the literal recurrence over each prefix (``oracle.recurrence``, explicit
  token matrices) read out with q_t, for the dense and KDA forms;
* delta-rule retrieval: alpha = beta = 1, unit keys and q_t = k_t give
  o_t = v_t;
* exact rational arithmetic (Fraction) over explicit matrices;
* segments are independent, the pair is the build's, outputs are linear in q,
  and the literal path equals the specialised one.
[the pair is cached at a segment's first prefill; remio.ai HYPIC article
(Japanese), section on how HYPIC composes linear-attention states]
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import DENSE, DIAG, KDA, SCALAR

CUTS = [0, 5, 5, 17, 40]


def _inputs(form, B, N, H, dk, dv, seed, unit_keys=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, N, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((B, N, H, dk))
    v = rng.standard_normal((B, N, H, dv))
    ashape = (B, N, H, dk) if form in (DIAG, KDA) else (B, N, H)
    a = rng.uniform(0.6, 1.0, size=ashape)
    b = rng.uniform(0.0, 1.0, size=(B, N, H)) if form in (DENSE, KDA) else None
    return q, k, v, a, b


@pytest.mark.parametrize("literal", [False, True])
def test_plain_linear_attention_is_masked_product(literal):
    q, k, v, _, _ = _inputs(SCALAR, 2, CUTS[-1], 3, 6, 5, 1, unit_keys=False)
    a = np.ones(q.shape[:3])
    out = oracle.prefill(SCALAR, q, k, v, a, None, CUTS, literal=literal)
    for lo, hi in zip(CUTS[:-1], CUTS[1:]):
        for b in range(2):
            for h in range(3):
                Q, K, V = q[b, lo:hi, h], k[b, lo:hi, h], v[b, lo:hi, h]
                want = np.tril(Q @ K.T) @ V
                assert np.allclose(out["O"][b, lo:hi, h], want, rtol=1e-12, atol=1e-12)


def test_scalar_decay_closed_form():
    q, k, v, a, _ = _inputs(SCALAR, 1, CUTS[-1], 2, 5, 4, 2, unit_keys=False)
    out = oracle.prefill(SCALAR, q, k, v, a, None, CUTS)
    for lo, hi in zip(CUTS[:-1], CUTS[1:]):
        for h in range(2):
            for t in range(lo, hi):
                want = np.zeros(4)
                for s in range(lo, t + 1):
                    w = np.prod(a[0, s + 1:t + 1, h])
                    want += w * np.dot(q[0, t, h], k[0, s, h]) * v[0, s, h]
                assert np.allclose(out["O"][0, t, h], want, rtol=1e-12, atol=1e-12)


def test_diagonal_gate_closed_form():
    q, k, v, a, _ = _inputs(DIAG, 1, CUTS[-1], 2, 5, 4, 3, unit_keys=False)
    out = oracle.prefill(DIAG, q, k, v, a, None, CUTS)
    for lo, hi in zip(CUTS[:-1], CUTS[1:]):
        for h in range(2):
            for t in range(lo, hi):
                want = np.zeros(4)
                for s in range(lo, t + 1):
                    w = np.prod(a[0, s + 1:t + 1, h], axis=0)  # per channel
                    want += np.dot(q[0, t, h] * w, k[0, s, h]) * v[0, s, h]
                assert np.allclose(out["O"][0, t, h], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("form", [DENSE, KDA])
def test_outputs_are_prefix_recurrences_read_out(form):
    """o_t = S_t^T q_t with S_t the literal recurrence over the segment's
    tokens up to t, from zero."""
    q, k, v, a, b = _inputs(form, 1, CUTS[-1], 2, 6, 5, 4)
    out = oracle.prefill(form, q, k, v, a, b, CUTS)
    for lo, hi in zip(CUTS[:-1], CUTS[1:]):
        for t in range(lo, hi):
            sl = slice(lo, t + 1)
            S = oracle.recurrence(form, k[:, sl], v[:, sl], a[:, sl], b[:, sl])  # [B, H, dk, dv]
            for h in range(2):
                want = S[0, h].T @ q[0, t, h]
                assert np.allclose(out["O"][0, t, h], want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("literal", [False, True])
def test_delta_rule_retrieval(literal):
    """alpha = beta = 1, unit keys, q_t = k_t: the delta rule writes v_t under
    k_t exactly, so the readout returns v_t."""
    _, k, v, _, _ = _inputs(DENSE, 1, 30, 2, 8, 6, 5)
    one = np.ones(k.shape[:3])
    out = oracle.prefill(DENSE, k, k, v, one, one, [0, 12, 30], literal=literal)
    assert np.allclose(out["O"], v, rtol=1e-10, atol=1e-10)


def _fraction_prefill(form, q, k, v, a, b, lo, hi):
    """Exact rationals over explicit matrices: T_t, S_t = T_t S_{t-1} + b k v^T,
    o_t = S_t^T q_t."""
    dk, dv = k.shape[-1], v.shape[-1]
    S = [[Fraction(0)] * dv for _ in range(dk)]
    outs = []
    for t in range(lo, hi):
        kt = [Fraction(x) for x in k[t]]
        bt = Fraction(b[t]) if b is not None else Fraction(1)
        if form == SCALAR:
            T = [[Fraction(a[t]) if i == j else Fraction(0) for j in range(dk)] for i in range(dk)]
        elif form == DIAG:
            T = [[Fraction(a[t][i]) if i == j else Fraction(0) for j in range(dk)] for i in range(dk)]
        elif form == DENSE:
            T = [[Fraction(a[t]) * ((1 if i == j else 0) - bt * kt[i] * kt[j]) for j in range(dk)]
                 for i in range(dk)]
        else:  # KDA: (I - b k k^T) Diag(a)
            T = [[((1 if i == j else 0) - bt * kt[i] * kt[j]) * Fraction(a[t][j]) for j in range(dk)]
                 for i in range(dk)]
        S = [[sum(T[i][l] * S[l][j] for l in range(dk)) + bt * kt[i] * Fraction(v[t][j])
              for j in range(dv)] for i in range(dk)]
        qt = [Fraction(x) for x in q[t]]
        outs.append([sum(qt[i] * S[i][j] for i in range(dk)) for j in range(dv)])
    return outs


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
@pytest.mark.parametrize("literal", [False, True])
def test_exact_rational_brute_force(form, literal):
    rng = np.random.default_rng(60 + form)
    dk, dv, N = 3, 2, 7
    dy = lambda shape: rng.integers(-4, 5, size=shape) / 8.0
    k, q, v = dy((1, N, 1, dk)), dy((1, N, 1, dk)), dy((1, N, 1, dv))
    ashape = (1, N, 1, dk) if form in (DIAG, KDA) else (1, N, 1)
    a = rng.integers(1, 5, size=ashape) / 4.0
    b = rng.integers(0, 5, size=(1, N, 1)) / 4.0 if form in (DENSE, KDA) else None
    cuts = [0, 3, 7]
    out = oracle.prefill(form, q, k, v, a, b, cuts, literal=literal)
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        want = _fraction_prefill(form, q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0],
                                 None if b is None else b[0, :, 0], lo, hi)
        for t, row in zip(range(lo, hi), want):
            got = out["O"][0, t, 0]
            for j in range(dv):
                assert abs(got[j] - float(row[j])) <= 1e-14 * max(1.0, abs(float(row[j])))


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
def test_segments_are_independent_and_pair_is_the_build(form):
    q, k, v, a, b = _inputs(form, 1, CUTS[-1], 2, 6, 5, 7)
    out = oracle.prefill(form, q, k, v, a, b, CUTS)
    ref = oracle.build(form, k, v, a, b, CUTS)
    for key in ref:
        assert np.array_equal(out[key], ref[key]), key
    # the last segment alone gives the same outputs
    lo, hi = CUTS[-2], CUTS[-1]
    sl = lambda x: None if x is None else x[:, lo:hi]
    alone = oracle.prefill(form, sl(q), sl(k), sl(v), sl(a), sl(b), [0, hi - lo])
    assert np.allclose(alone["O"], out["O"][:, lo:hi], rtol=1e-13, atol=1e-14)
    # perturbing the first segment leaves the others' outputs unchanged
    k2 = k.copy()
    k2[:, :CUTS[1]] *= -1.0
    out2 = oracle.prefill(form, q, k2, v, a, b, CUTS)
    assert np.array_equal(out2["O"][:, CUTS[1]:], out["O"][:, CUTS[1]:])


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
def test_literal_equals_specialised_and_linear_in_q(form):
    q, k, v, a, b = _inputs(form, 2, CUTS[-1], 2, 5, 4, 8)
    fast = oracle.prefill(form, q, k, v, a, b, CUTS)
    slow = oracle.prefill(form, q, k, v, a, b, CUTS, literal=True)
    assert np.allclose(fast["O"], slow["O"], rtol=1e-11, atol=1e-12)
    q2 = np.random.default_rng(9).standard_normal(q.shape)
    o2 = oracle.prefill(form, q2, k, v, a, b, CUTS)["O"]
    o12 = oracle.prefill(form, 2.0 * q - 3.0 * q2, k, v, a, b, CUTS)["O"]
    assert np.allclose(o12, 2.0 * fast["O"] - 3.0 * o2, rtol=1e-11, atol=1e-11)
