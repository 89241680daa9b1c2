"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own update rule: each compares it with a
different computation of the same quantity (hand-worked exact values, closed
forms, exact rational brute force over explicit matrix products, invariants
of the composition identity, or a textbook routine in a special case).

Sources: HYPIC, xix.ai article (French), paragraph on linear layers (T_C as
the product of token transitions, S(C|0), the composition identity
S(C1.C2) = T(C2) S(C1) + S(C2), prefix independence, naive addition valid
only for plain linear attention); remio.ai article (Japanese), section on how
HYPIC composes linear-attention states (scalar / diagonal / dense forms).
"""
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import DENSE, DIAG, SCALAR
from tests.conftest import rel_fro, rel_fro_units

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(form, B, H, dk, dv, N, seed, alpha_range=(0.5, 1.0), beta_range=(0.0, 1.0),
                normalise=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, N, H, dk))
    if normalise:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, H, dv))
    ashape = (B, N, H, dk) if form == DIAG else (B, N, H)
    alpha = rng.uniform(*alpha_range, size=ashape)
    beta = rng.uniform(*beta_range, size=(B, N, H)) if form == DENSE else None
    return k, v, alpha, beta


def plain_T(form, res):
    """Plain T_C from the split form (lam, That)."""
    lam = res["lam"]
    if form == DENSE:
        return np.exp(lam)[..., None, None] * res["That"]
    dk = res["S"].shape[-2]
    eye = np.eye(dk)
    if form == SCALAR:
        return np.exp(lam)[..., None, None] * eye
    return np.exp(lam)[..., :, None] * eye


# --------------------------------------------------------------------------
# hand-worked golden examples (tests/golden/hand_examples.txt)
# --------------------------------------------------------------------------

def _parse_vec(s):
    return [Fraction(x.strip()) for x in s.split(",")]


def _parse_mat(s):
    return [_parse_vec(r) for r in s.split(";")]


def load_hand_examples():
    path = os.path.join(HERE, "golden", "hand_examples.txt")
    exs, cur = [], None
    for raw in open(path, encoding="utf-8"):
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("example"):
            m = re.match(r"example (\S+) form=(\S+) dk=(\d+) dv=(\d+)", line)
            cur = {"name": m.group(1), "form": {"scalar": SCALAR, "diag": DIAG,
                                                 "dense": DENSE}[m.group(2)],
                   "dk": int(m.group(3)), "dv": int(m.group(4)), "tokens": []}
        elif line.startswith("token"):
            fields = dict(f.split("=") for f in line.split()[1:])
            cur["tokens"].append({key: _parse_vec(val) for key, val in fields.items()})
        elif line == "end":
            exs.append(cur)
            cur = None
        else:
            key, val = (x.strip() for x in line.split("=", 1))
            if key == "lam":
                cur[key] = [sum(np.log(float(Fraction(a))) for a in re.findall(r"ln\(([^)]*)\)", c))
                            for c in val.split(",")]
            else:
                cur[key] = _parse_mat(val)
    return exs


HAND = load_hand_examples()


@pytest.mark.parametrize("ex", HAND, ids=[e["name"] for e in HAND])
@pytest.mark.parametrize("literal", [False, True])
def test_hand_examples(ex, literal):
    form, dk, dv = ex["form"], ex["dk"], ex["dv"]
    toks = ex["tokens"]
    N = len(toks)
    k = np.array([[[float(x) for x in t["k"]]] for t in toks])[None]
    v = np.array([[[float(x) for x in t["v"]]] for t in toks])[None]
    if form == DIAG:
        alpha = np.array([[[float(x) for x in t["alpha"]]] for t in toks])[None]
    else:
        alpha = np.array([[float(t["alpha"][0])] for t in toks])[None]
    beta = np.array([[float(t["beta"][0])] for t in toks])[None]
    res = oracle.build(form, k, v, alpha, beta, [0, N], literal=literal, want_T=True)
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    # dyadic values: exact in fp64
    assert np.array_equal(res["S"][0, 0, 0], f(ex["S"]))
    assert np.array_equal(res["T"][0, 0, 0], f(ex["T"]))
    if form == DENSE:
        assert np.array_equal(res["That"][0, 0, 0], f(ex["That"]))
    np.testing.assert_allclose(np.ravel(res["lam"][0, 0, 0]), ex["lam"], rtol=1e-15, atol=1e-15)
    S_in = f(ex["S_in"])[None, None, None]
    comp = oracle.compose(form, res["lam"], res.get("That"), res["S"], [0, 1], [0], S_in)
    np.testing.assert_allclose(comp[0, 0, 0], f(ex["composed"]), rtol=0, atol=1e-15)
    naive = oracle.naive_add(res["S"], [0, 1], [0], S_in)
    assert np.array_equal(naive[0, 0, 0], f(ex["naive"]))
    # token-by-token from S_in reaches the composed state too
    rec = oracle.recurrence(form, k, v, alpha, beta, S_in[0])
    np.testing.assert_allclose(rec[0, 0], f(ex["composed"]), rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# P1: split + compose equals the unsplit recurrence
# --------------------------------------------------------------------------

@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
@pytest.mark.parametrize("cuts", [[0, 63, 127], [0, 64, 128], [0, 65, 129], [0, 1, 40, 41, 90],
                                  [0, 0, 30, 30, 77]])
def test_p1_split_compose_equals_unsplit(form, cuts):
    B, H, dk, dv = 2, 2, 8, 6
    N = cuts[-1]
    k, v, alpha, beta = rand_inputs(form, B, H, dk, dv, N, seed=11 + len(cuts) + form,
                                    alpha_range=(0.8, 1.0))
    S_in = np.random.default_rng(5).standard_normal((1, B, H, dk, dv))
    res = oracle.build(form, k, v, alpha, beta, cuts)
    n_seg = len(cuts) - 1
    comp = oracle.compose(form, res["lam"], res.get("That"), res["S"], [0, n_seg],
                          list(range(n_seg)), S_in)
    ref = oracle.recurrence(form, k, v, alpha, beta, S_in[0])
    assert rel_fro(comp[0], ref) < 1e-12
    # and from a zero start
    comp0 = oracle.compose(form, res["lam"], res.get("That"), res["S"], [0, n_seg],
                           list(range(n_seg)))
    ref0 = oracle.recurrence(form, k, v, alpha, beta)
    assert rel_fro(comp0[0], ref0) < 1e-12


# --------------------------------------------------------------------------
# literal (explicit dense T_t products) vs specialised paths
# --------------------------------------------------------------------------

@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
def test_literal_equals_specialised(form):
    B, H, dk, dv = 1, 3, 8, 5
    cuts = [0, 17, 17, 50]
    k, v, alpha, beta = rand_inputs(form, B, H, dk, dv, cuts[-1], seed=3 + form)
    lit = oracle.build(form, k, v, alpha, beta, cuts, literal=True)
    fast = oracle.build(form, k, v, alpha, beta, cuts, want_T=True)
    assert rel_fro_units(fast["S"], lit["S"]) < 1e-13
    assert rel_fro_units(fast["T"], lit["T"]) < 1e-13
    np.testing.assert_allclose(fast["lam"], lit["lam"], rtol=1e-15, atol=1e-15)
    if form == DENSE:
        assert rel_fro_units(fast["That"], lit["That"]) < 1e-13
    # split form (lam, That) is the plain operator
    assert rel_fro_units(plain_T(form, lit), lit["T"]) < 1e-13


# --------------------------------------------------------------------------
# P2: identity transitions
# --------------------------------------------------------------------------

@pytest.mark.parametrize("literal", [False, True])
def test_p2_identity_dense(literal):
    B, H, dk, dv, N = 1, 2, 6, 4, 20
    k, v, _, _ = rand_inputs(DENSE, B, H, dk, dv, N, seed=2)
    alpha = np.ones((B, N, H))
    beta = np.zeros((B, N, H))
    res = oracle.build(DENSE, k, v, alpha, beta, [0, 7, N], literal=literal, want_T=True)
    eye = np.broadcast_to(np.eye(dk), res["That"].shape)
    assert np.array_equal(res["That"], eye)
    assert np.array_equal(res["T"], eye)
    assert np.all(res["lam"] == 0.0)
    assert np.all(res["S"] == 0.0)


def test_empty_segment_is_identity_pair():
    for form in (SCALAR, DIAG, DENSE):
        k, v, alpha, beta = rand_inputs(form, 1, 2, 4, 3, 10, seed=9)
        res = oracle.build(form, k, v, alpha, beta, [0, 0, 10, 10], want_T=True)
        for s in (0, 2):
            assert np.all(res["S"][s] == 0.0)
            assert np.all(res["lam"][s] == 0.0)
            assert np.array_equal(res["T"][s], np.broadcast_to(np.eye(4), res["T"][s].shape))


# --------------------------------------------------------------------------
# P3: plain linear attention -- S = K^T V, naive add == composition
# --------------------------------------------------------------------------

def test_p3_vanilla_linear_attention():
    B, H, dk, dv, N = 1, 2, 7, 5, 33
    k, v, _, _ = rand_inputs(SCALAR, B, H, dk, dv, N, seed=4, normalise=False)
    alpha = np.ones((B, N, H))
    cuts = [0, 10, 33]
    res = oracle.build(SCALAR, k, v, alpha, None, cuts)
    for s in range(2):
        for h in range(H):
            K = k[0, cuts[s]:cuts[s + 1], h]
            V = v[0, cuts[s]:cuts[s + 1], h]
            np.testing.assert_allclose(res["S"][s, 0, h], K.T @ V, rtol=1e-13, atol=1e-13)
    S_in = np.random.default_rng(1).standard_normal((1, B, H, dk, dv))
    comp = oracle.compose(SCALAR, res["lam"], None, res["S"], [0, 2], [0, 1], S_in)
    naive = oracle.naive_add(res["S"], [0, 2], [0, 1], S_in)
    assert np.array_equal(comp, naive)  # T = e^0 I = I exactly


# --------------------------------------------------------------------------
# P4 / P5: closed forms of the scalar and diagonal families
# --------------------------------------------------------------------------

def test_p4_scalar_closed_form():
    B, H, dk, dv, N = 1, 3, 6, 4, 40
    k, v, alpha, _ = rand_inputs(SCALAR, B, H, dk, dv, N, seed=6, normalise=False)
    res = oracle.build(SCALAR, k, v, alpha, None, [0, N], want_T=True)
    for h in range(H):
        a = alpha[0, :, h]
        # w_t = prod_{s>t} a_s  (suffix products, computed right to left)
        w = np.ones(N)
        for t in range(N - 2, -1, -1):
            w[t] = w[t + 1] * a[t + 1]
        S = np.einsum("t,ti,tj->ij", w, k[0, :, h], v[0, :, h])
        np.testing.assert_allclose(res["S"][0, 0, h], S, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(res["T"][0, 0, h], np.prod(a) * np.eye(dk), rtol=1e-12,
                                   atol=0)
        np.testing.assert_allclose(res["lam"][0, 0, h], np.log(np.prod(a)), rtol=1e-12)


def test_p5_diag_closed_form():
    B, H, dk, dv, N = 1, 2, 5, 3, 30
    k, v, alpha, _ = rand_inputs(DIAG, B, H, dk, dv, N, seed=8, normalise=False)
    res = oracle.build(DIAG, k, v, alpha, None, [0, N], want_T=True)
    for h in range(H):
        for i in range(dk):
            a = alpha[0, :, h, i]
            w = np.array([np.prod(a[t + 1:]) for t in range(N)])
            row = (w * k[0, :, h, i]) @ v[0, :, h]
            np.testing.assert_allclose(res["S"][0, 0, h, i], row, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(res["T"][0, 0, h, i, i], np.prod(a), rtol=1e-12)
        off = res["T"][0, 0, h] - np.diag(np.diag(res["T"][0, 0, h]))
        assert np.all(off == 0.0)


# --------------------------------------------------------------------------
# P6: associativity; the chain's pair equals the pair of the concatenation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
def test_p6_associativity(form):
    B, H, dk, dv = 1, 2, 6, 4
    cuts = [0, 9, 21, 30, 44]
    k, v, alpha, beta = rand_inputs(form, B, H, dk, dv, cuts[-1], seed=21 + form,
                                    alpha_range=(0.7, 1.0))
    res = oracle.build(form, k, v, alpha, beta, cuts)
    That = res.get("That")
    S_in = np.random.default_rng(7).standard_normal((1, B, H, dk, dv))
    seq = oracle.compose(form, res["lam"], That, res["S"], [0, 4], [0, 1, 2, 3], S_in)
    # (p2 o p1) as one pair, then p3, p4
    S12, l12, T12 = oracle.compose(form, res["lam"], That, res["S"], [0, 2], [0, 1],
                                   want_pair=True)
    # the chain's pair is the pair of the concatenated tokens built directly
    n2 = cuts[2]
    whole = oracle.build(form, k[:, :n2], v[:, :n2], alpha[:, :n2],
                         None if beta is None else beta[:, :n2], [0, n2])
    assert rel_fro_units(S12[0], whole["S"][0]) < 1e-12
    np.testing.assert_allclose(l12[0], whole["lam"][0], rtol=1e-13)
    if form == DENSE:
        assert rel_fro_units(T12[0], whole["That"][0]) < 1e-12
    pool_lam = np.concatenate([l12, res["lam"][2:]])
    pool_S = np.concatenate([S12, res["S"][2:]])
    pool_T = np.concatenate([T12, That[2:]]) if form == DENSE else None
    left = oracle.compose(form, pool_lam, pool_T, pool_S, [0, 3], [0, 1, 2], S_in)
    assert rel_fro(left, seq) < 1e-12
    # p1 then (p4 o p3 o p2)
    S234, l234, T234 = oracle.compose(form, res["lam"], That, res["S"], [0, 3], [1, 2, 3],
                                      want_pair=True)
    pool_lam = np.concatenate([res["lam"][:1], l234])
    pool_S = np.concatenate([res["S"][:1], S234])
    pool_T = np.concatenate([That[:1], T234]) if form == DENSE else None
    right = oracle.compose(form, pool_lam, pool_T, pool_S, [0, 2], [0, 1], S_in)
    assert rel_fro(right, seq) < 1e-12


# --------------------------------------------------------------------------
# P7: naive error is exactly the omitted (I - T(C2)) S(C1)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
def test_p7_naive_error(form):
    B, H, dk, dv = 1, 2, 6, 5
    cuts = [0, 25, 50]
    k, v, alpha, beta = rand_inputs(form, B, H, dk, dv, cuts[-1], seed=31 + form,
                                    alpha_range=(0.9, 1.0))
    res = oracle.build(form, k, v, alpha, beta, cuts, want_T=True)
    comp = oracle.compose(form, res["lam"], res.get("That"), res["S"], [0, 2], [0, 1])
    naive = oracle.naive_add(res["S"], [0, 2], [0, 1])
    T2 = res["T"][1]
    S1 = res["S"][0]
    expect = np.einsum("bhij,bhjk->bhik", np.eye(dk) - T2, S1)
    np.testing.assert_allclose(naive[0] - comp[0], expect, rtol=1e-11, atol=1e-12)
    # and it does not vanish unless T(C2) = I
    assert rel_fro(naive[0], comp[0]) > 1e-3


# --------------------------------------------------------------------------
# P8: prefix independence of the pair
# --------------------------------------------------------------------------

@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
def test_p8_prefix_independence(form):
    B, H, dk, dv = 1, 2, 5, 4
    k, v, alpha, beta = rand_inputs(form, B, H, dk, dv, 50, seed=41 + form)
    alone = oracle.build(form, k[:, 20:], v[:, 20:], alpha[:, 20:],
                         None if beta is None else beta[:, 20:], [0, 30])
    after = oracle.build(form, k, v, alpha, beta, [0, 20, 50])
    # different preceding tokens
    k2, v2, a2, b2 = rand_inputs(form, B, H, dk, dv, 20, seed=99)
    kk = np.concatenate([k2, k[:, 20:]], axis=1)
    vv = np.concatenate([v2, v[:, 20:]], axis=1)
    aa = np.concatenate([a2, alpha[:, 20:]], axis=1)
    bb = None if beta is None else np.concatenate([b2, beta[:, 20:]], axis=1)
    other = oracle.build(form, kk, vv, aa, bb, [0, 20, 50])
    for res in (after, other):
        assert np.array_equal(res["S"][1], alone["S"][0])
        assert np.array_equal(res["lam"][1], alone["lam"][0])
        if form == DENSE:
            assert np.array_equal(res["That"][1], alone["That"][0])


# --------------------------------------------------------------------------
# P9: delta-rule retrieval
# --------------------------------------------------------------------------

def test_p9_delta_rule_retrieval():
    B, H, dk, dv, N = 1, 2, 8, 6, 12
    k, v, _, _ = rand_inputs(DENSE, B, H, dk, dv, N, seed=51)
    alpha = np.ones((B, N, H))
    beta = np.ones((B, N, H))
    for L in (1, 5, N):
        res = oracle.build(DENSE, k[:, :L], v[:, :L], alpha[:, :L], beta[:, :L], [0, L])
        for h in range(H):
            got = res["S"][0, 0, h].T @ k[0, L - 1, h]
            np.testing.assert_allclose(got, v[0, L - 1, h], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P10: exact rational brute force over explicit matrix products
# --------------------------------------------------------------------------

def _frac_transition(form, k, a, b):
    d = len(k)
    T = [[Fraction(0)] * d for _ in range(d)]
    for i in range(d):
        for j in range(d):
            eye = Fraction(int(i == j))
            if form == SCALAR:
                T[i][j] = a[0] * eye
            elif form == DIAG:
                T[i][j] = a[i] * eye
            else:
                T[i][j] = a[0] * (eye - b * k[i] * k[j])
    return T


def _fmat(A, B):
    return [[sum(A[i][l] * B[l][j] for l in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p10_exact_rational_brute_force(form, seed):
    """T_C as the explicit product T_L ... T_1, and S(C|0) as the unrolled sum
    sum_t (T_L ... T_{t+1}) U_t, in exact rationals; the fp64 oracle must agree
    to fp64 rounding."""
    rng = np.random.default_rng(1000 + seed)
    dk, dv, L = 3, 2, 6
    dy = lambda shape, lo, hi: rng.integers(lo, hi, size=shape) / 8.0  # dyadic
    k = dy((L, dk), -8, 9)
    v = dy((L, dv), -8, 9)
    alpha = rng.integers(1, 9, size=(L, dk if form == DIAG else 1)) / 8.0
    beta = rng.integers(0, 9, size=L) / 8.0
    Fk = [[Fraction(x) for x in r] for r in k]
    Fv = [[Fraction(x) for x in r] for r in v]
    Fa = [[Fraction(x) for x in r] for r in alpha]
    Fb = [Fraction(x) if form == DENSE else Fraction(1) for x in beta]
    Ts = [_frac_transition(form, Fk[t], Fa[t], Fb[t]) for t in range(L)]
    eye = [[Fraction(int(i == j)) for j in range(dk)] for i in range(dk)]
    T = eye
    for t in range(L):
        T = _fmat(Ts[t], T)
    S = [[Fraction(0)] * dv for _ in range(dk)]
    for t in range(L):
        suffix = eye
        for s in range(t + 1, L):
            suffix = _fmat(Ts[s], suffix)
        U = [[Fb[t] * Fk[t][i] * Fv[t][j] for j in range(dv)] for i in range(dk)]
        SU = _fmat(suffix, U)
        S = [[S[i][j] + SU[i][j] for j in range(dv)] for i in range(dk)]
    ak = alpha[None, :, None, :] if form == DIAG else alpha[None, :, None, 0]
    for literal in (False, True):
        res = oracle.build(form, k[None, :, None], v[None, :, None], ak, beta[None, :, None],
                           [0, L], literal=literal, want_T=True)
        exactS = np.array([[float(x) for x in r] for r in S])
        exactT = np.array([[float(x) for x in r] for r in T])
        scale = max(1.0, np.abs(exactS).max())
        assert np.abs(res["S"][0, 0, 0] - exactS).max() <= 1e-14 * scale
        assert np.abs(res["T"][0, 0, 0] - exactT).max() <= 1e-15


# --------------------------------------------------------------------------
# P11: one-hot keys -- closed form of the dense build
# --------------------------------------------------------------------------

def one_hot_inputs(dk, dv, N, H, seed):
    """k_t = e_{j_t}, beta = 1, alpha_t = 2^{-m_t}, m_t = 1 on ~1/16 of the
    tokens, small integer v.  Every quantity of the chunked build is exact."""
    rng = np.random.default_rng(seed)
    j = rng.integers(0, dk, size=(N, H))
    k = np.zeros((1, N, H, dk))
    for t in range(N):
        for h in range(H):
            k[0, t, h, j[t, h]] = 1.0
    v = rng.integers(-8, 8, size=(1, N, H, dv)).astype(np.float64)
    m = (rng.random((N, H)) < 1.0 / 16).astype(np.float64)
    alpha = (2.0 ** (-m))[None]
    beta = np.ones((1, N, H))
    return k, v, alpha, beta, j


def one_hot_expected(k, v, alpha, j, lo, hi):
    """S[j] = (prod_{s>t_j} a_s) v_{t_j} for the last token t_j keyed j (0 if
    none); That = Diag(1[j not keyed]); lam = sum ln a."""
    _, N, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv))
    That = np.zeros((H, dk, dk))
    lam = np.zeros(H)
    for h in range(H):
        keyed = set()
        for row in range(dk):
            ts = [t for t in range(lo, hi) if j[t, h] == row]
            if ts:
                tj = ts[-1]
                keyed.add(row)
                S[h, row] = np.prod(alpha[0, tj + 1:hi, h]) * v[0, tj, h]
        for row in range(dk):
            That[h, row, row] = 0.0 if row in keyed else 1.0
        lam[h] = np.sum(np.log(alpha[0, lo:hi, h]))
    return S, That, lam


def test_p11_one_hot_closed_form():
    dk, dv, H = 16, 8, 2
    cuts = [0, 63, 64 + 63, 64 + 63 + 200]
    N = cuts[-1]
    k, v, alpha, beta, j = one_hot_inputs(dk, dv, N, H, seed=61)
    res = oracle.build(DENSE, k, v, alpha, beta, cuts)
    for s in range(len(cuts) - 1):
        S, That, lam = one_hot_expected(k, v, alpha, j, cuts[s], cuts[s + 1])
        assert np.array_equal(res["S"][s, 0], S)
        assert np.array_equal(res["That"][s, 0], That)
        np.testing.assert_allclose(res["lam"][s, 0], lam, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# P12: permutation-marker chains -- exact bookkeeping of compose
# --------------------------------------------------------------------------

def test_p12_permutation_chain():
    rng = np.random.default_rng(71)
    P, B, H, d = 12, 2, 3, 6
    perms = np.array([[[rng.permutation(d) for _ in range(H)] for _ in range(B)]
                      for _ in range(P)])
    That = np.zeros((P, B, H, d, d))
    for p in range(P):
        for b in range(B):
            for h in range(H):
                That[p, b, h, np.arange(d), perms[p, b, h]] = 1.0
    lam = np.zeros((P, B, H))
    S = rng.integers(-4, 5, size=(P, B, H, d, d)).astype(np.float64)
    off = [0, 5, 5, 12]
    idx = [3, 0, 7, 7, 11, 1, 2, 3, 4, 5, 6, 9]
    S_in = rng.integers(-4, 5, size=(3, B, H, d, d)).astype(np.float64)
    out = oracle.compose(DENSE, lam, That, S, off, idx, S_in)
    for r in range(3):
        cur = S_in[r].copy()
        for p in idx[off[r]:off[r + 1]]:
            # (Perm S)[i] = S[perm[i]]
            nxt = np.empty_like(cur)
            for b in range(B):
                for h in range(H):
                    nxt[b, h] = cur[b, h][perms[p, b, h]]
            cur = nxt + S[p]
        assert np.array_equal(out[r], cur)


# --------------------------------------------------------------------------
# argument checks
# --------------------------------------------------------------------------

def test_oracle_rejects_bad_offsets_and_chains():
    k, v, alpha, beta = rand_inputs(DENSE, 1, 1, 4, 4, 10, seed=1)
    with pytest.raises(ValueError):
        oracle.build(DENSE, k, v, alpha, beta, [0, 6, 5, 10])
    with pytest.raises(ValueError):
        oracle.build(DENSE, k, v, alpha, beta, [0, 9])
    res = oracle.build(DENSE, k, v, alpha, beta, [0, 10])
    with pytest.raises(ValueError):
        oracle.compose(DENSE, res["lam"], res["That"], res["S"], [0, 1], [1])
