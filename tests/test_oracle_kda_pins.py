"""Pins of the oracle's dense delta form with per-channel gates (KDA form):
T_t = (I - beta_t k_t k_t^T) Diag(alpha_t), alpha_t in (0, 1]^dk.
[xix.ai HYPIC article (French), paragraph on linear layers: the families whose
transitions are composed include KDA; T_C is the product of the segment's
token transitions.]

Split of the pair: lambda_C = sum_t ln m_t with m_t = max_i alpha_t,i, and
That_C = prod_t (I - beta_t k_t k_t^T) Diag(alpha_t / m_t), so that
T_C = e^{lambda_C} That_C (the dense GDN split when all channels share a gate).

Each pin compares the oracle with a different computation: the dense GDN form
and the diagonal form in the special cases that reduce to them, exact rational
products of explicit matrices, the literal path, and the unsplit recurrence.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import DENSE, DIAG, KDA
from tests.conftest import rel_fro


def kda_inputs(B, H, dk, dv, N, seed, alpha=(0.5, 1.0), beta=(0.0, 1.0)):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, H, dv))
    a = rng.uniform(*alpha, size=(B, N, H, dk))
    b = rng.uniform(*beta, size=(B, N, H))
    return k, v, a, b


def test_kda_literal_equals_specialised():
    k, v, a, b = kda_inputs(2, 2, 6, 5, 40, seed=1)
    offs = [0, 7, 7, 23, 40]
    lit = oracle.build(KDA, k, v, a, b, offs, literal=True)
    spe = oracle.build(KDA, k, v, a, b, offs, want_T=True)
    for key in ("S", "That", "T"):
        assert rel_fro(spe[key], lit[key]) <= 1e-12, key
    assert np.max(np.abs(spe["lam"] - lit["lam"])) <= 1e-12


@pytest.mark.parametrize("literal", [False, True])
def test_kda_with_shared_gates_is_dense_gdn(literal):
    """alpha_t,i = alpha_t for every channel: T_t = alpha_t (I - b k k^T)."""
    k, v, a, b = kda_inputs(1, 3, 8, 6, 30, seed=2)
    a1 = a[..., 0]
    a_all = np.repeat(a1[..., None], 8, axis=-1)
    offs = [0, 13, 30]
    kda = oracle.build(KDA, k, v, a_all, b, offs, literal=literal, want_T=True)
    gdn = oracle.build(DENSE, k, v, a1, b, offs, literal=literal, want_T=True)
    for key in ("S", "That", "T"):
        assert rel_fro(kda[key], gdn[key]) <= 1e-12, key
    assert np.max(np.abs(kda["lam"] - gdn["lam"])) <= 1e-12


def test_kda_without_erase_is_diagonal():
    """beta = 0: T_t = Diag(alpha_t), no erase term."""
    k, v, a, _ = kda_inputs(1, 2, 6, 4, 25, seed=3)
    zero = np.zeros(a.shape[:3])
    offs = [0, 9, 25]
    kda = oracle.build(KDA, k, v, a, zero, offs, want_T=True)
    dia = oracle.build(DIAG, k, v, a, None, offs, want_T=True)
    # beta = 0 also drops the write term of the KDA form (b k v^T)
    assert np.max(np.abs(kda["S"])) == 0.0
    assert rel_fro(kda["T"], dia["T"]) <= 1e-12
    for s in range(2):
        m = np.max(a[0, offs[s]:offs[s + 1]], axis=-1)          # [L, H]
        want_lam = np.sum(np.log(m), axis=0)
        assert np.max(np.abs(kda["lam"][s, 0] - want_lam)) <= 1e-12
        ratio = np.prod(a[0, offs[s]:offs[s + 1]] / m[..., None], axis=0)  # [H, dk]
        for h in range(2):
            np.testing.assert_allclose(kda["That"][s, 0, h], np.diag(ratio[h]), atol=1e-14)


def _fmat(A, B):
    return [[sum(A[i][l] * B[l][j] for l in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kda_exact_rational(seed):
    """T_C as the explicit product T_L ... T_1 and S(C|0) token by token, in
    exact rationals; That_C = T_C / prod m_t."""
    rng = np.random.default_rng(700 + seed)
    dk, dv, L = 3, 2, 6
    k = rng.integers(-8, 9, size=(L, dk)) / 8.0
    v = rng.integers(-8, 9, size=(L, dv)) / 8.0
    a = rng.integers(1, 9, size=(L, dk)) / 8.0
    b = rng.integers(0, 9, size=L) / 8.0
    F = lambda x: Fraction(x)
    T = [[Fraction(int(i == j)) for j in range(dk)] for i in range(dk)]
    S = [[Fraction(0)] * dv for _ in range(dk)]
    M = Fraction(1)
    for t in range(L):
        Tt = [[(Fraction(int(i == j)) - F(b[t]) * F(k[t, i]) * F(k[t, j])) * F(a[t, j])
               for j in range(dk)] for i in range(dk)]
        T = _fmat(Tt, T)
        TS = _fmat(Tt, S)
        S = [[TS[i][j] + F(b[t]) * F(k[t, i]) * F(v[t, j]) for j in range(dv)] for i in range(dk)]
        M *= F(max(a[t]))
    exact_T = np.array([[float(x) for x in r] for r in T])
    exact_S = np.array([[float(x) for x in r] for r in S])
    exact_Th = np.array([[float(x / M) for x in r] for r in T])
    for literal in (False, True):
        res = oracle.build(KDA, k[None, :, None], v[None, :, None], a[None, :, None],
                           b[None, :, None], [0, L], literal=literal, want_T=True)
        assert np.abs(res["T"][0, 0, 0] - exact_T).max() <= 1e-15
        assert np.abs(res["S"][0, 0, 0] - exact_S).max() <= 1e-14 * max(1.0, np.abs(exact_S).max())
        assert np.abs(res["That"][0, 0, 0] - exact_Th).max() <= 1e-14
        assert abs(res["lam"][0, 0, 0] - float(np.sum(np.log(np.max(a, axis=1))))) <= 1e-13


@pytest.mark.parametrize("cuts", [[0, 9, 10, 31], [0, 1, 17, 40], [0, 0, 20, 20, 33]])
def test_kda_split_compose_equals_unsplit(cuts):
    k, v, a, b = kda_inputs(2, 2, 6, 5, cuts[-1], seed=4)
    pairs = oracle.build(KDA, k, v, a, b, cuts)
    n = len(cuts) - 1
    rng = np.random.default_rng(9)
    S_in = rng.standard_normal((1, 2, 2, 6, 5))
    got = oracle.compose(KDA, pairs["lam"], pairs["That"], pairs["S"], [0, n], list(range(n)),
                         S_in)
    ref = oracle.recurrence(KDA, k, v, a, b, S_in[0])
    assert rel_fro(got[0], ref) <= 1e-12
    # the chain's own pair is the pair of the concatenated tokens
    _, lam_c, That_c = oracle.compose(KDA, pairs["lam"], pairs["That"], pairs["S"], [0, n],
                                      list(range(n)), want_pair=True)
    whole = oracle.build(KDA, k, v, a, b, [0, cuts[-1]])
    assert rel_fro(That_c[0], whole["That"][0]) <= 1e-12
    assert np.max(np.abs(lam_c[0] - whole["lam"][0])) <= 1e-12


def test_kda_That_is_bounded():
    """beta |k|^2 <= 2 and gates scaled by their maximum: ||That||_2 <= 1."""
    k, v, a, b = kda_inputs(1, 3, 8, 4, 200, seed=5, alpha=(0.05, 1.0))
    res = oracle.build(KDA, k, v, a, b, [0, 200])
    for h in range(3):
        assert np.linalg.norm(res["That"][0, 0, h], 2) <= 1.0 + 1e-12
