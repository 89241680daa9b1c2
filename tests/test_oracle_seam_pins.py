"""Pins of the oracle's reuse with seam windows (``oracle.seam_compose``).

On reuse, the first w tokens of an inner segment are kept out of its cached
pair and run again from the running state, each emitting its layer output;
then the pair of the rest of the segment is applied.  [xix.ai HYPIC article
(French), paragraph on full-attention layers: seam windows of w tokens (8 by
default) at the start of each inner segment, recomputed under the full prefix;
the linear layers advance the running state through them and pass each
token's output up.]  The readout is o_t = S_t^T q_t with S_t the state after
token t.

None of these re-types the oracle's update: each compares it with another
computation of the same quantity -- the unsplit per-token recurrence over the
whole prompt (a different routine of the oracle, itself pinned), the
delta-rule retrieval identity, exact rational arithmetic over explicit
matrices, or plain composition when every window is empty.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import DENSE, DIAG, KDA, SCALAR
from tests.conftest import rel_fro


def _inputs(form, B, H, dk, dv, N, seed, alpha_range=(0.6, 1.0)):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((B, N, H, dk))
    v = rng.standard_normal((B, N, H, dv))
    alpha = rng.uniform(*alpha_range, size=(B, N, H, dk) if form in (DIAG, KDA) else (B, N, H))
    beta = rng.uniform(0.0, 1.0, size=(B, N, H)) if form in (DENSE, KDA) else None
    return q, k, v, alpha, beta


def split_prompt(seg_lens, seam_lens):
    """Token ranges of a prompt cut into segments; segment i's first
    seam_lens[i] tokens form its seam window, the rest its cached part.
    Returns (seam token positions in order, remainder offsets over the
    concatenated remainders, seam offsets per segment, remainder positions)."""
    seam_pos, rem_pos, seam_off, rem_off = [], [], [0], [0]
    start = 0
    for L, w in zip(seg_lens, seam_lens):
        w = min(w, L)
        seam_pos += list(range(start, start + w))
        rem_pos += list(range(start + w, start + L))
        seam_off.append(len(seam_pos))
        rem_off.append(len(rem_pos))
        start += L
    return np.array(seam_pos, dtype=np.int64), rem_off, seam_off, np.array(rem_pos, dtype=np.int64)


def _take(x, pos):
    return None if x is None else x[:, pos]


def run_split(form, seg_lens, seam_lens, B=2, H=2, dk=6, dv=5, seed=0, literal=False,
              with_S_in=True):
    N = int(sum(seg_lens))
    q, k, v, alpha, beta = _inputs(form, B, H, dk, dv, N, seed)
    seam_pos, rem_off, seam_off, rem_pos = split_prompt(seg_lens, seam_lens)
    pool = oracle.build(form, _take(k, rem_pos), _take(v, rem_pos), _take(alpha, rem_pos),
                        _take(beta, rem_pos), rem_off, literal=literal)
    rng = np.random.default_rng(seed + 99)
    S_in = rng.standard_normal((1, B, H, dk, dv)) if with_S_in else None
    n = len(seg_lens)
    S_out, O = oracle.seam_compose(form, pool["lam"], pool.get("That"), pool["S"], [0, n],
                                   list(range(n)), seam_off, _take(q, seam_pos),
                                   _take(k, seam_pos), _take(v, seam_pos),
                                   _take(alpha, seam_pos), _take(beta, seam_pos), S_in,
                                   literal=literal)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S_in=S_in, S_out=S_out, O=O,
                seam_pos=seam_pos, N=N)


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
@pytest.mark.parametrize("literal", [False, True])
@pytest.mark.parametrize("seg_lens,seam_lens", [
    ([7, 9, 5], [0, 3, 3]),
    ([4, 10, 3, 8], [0, 8, 8, 2]),      # a window covering its whole segment
    ([12, 1, 6], [2, 1, 0]),            # a one-token segment that is all seam
])
def test_seam_split_equals_unsplit(form, literal, seg_lens, seam_lens):
    """Seam windows plus the pairs of the segments' remainders reproduce the
    unsplit recurrence over the whole prompt: the final state, and every seam
    token's output equals the unsplit state after that token times q."""
    r = run_split(form, seg_lens, seam_lens, literal=literal)
    k, v, alpha, beta, q, S_in = r["k"], r["v"], r["alpha"], r["beta"], r["q"], r["S_in"]
    S_in0 = S_in[0]
    ref = oracle.recurrence(form, k, v, alpha, beta, S_in0)
    assert rel_fro(r["S_out"][0], ref) <= 1e-12
    for i, p in enumerate(r["seam_pos"]):
        Sp = oracle.recurrence(form, k[:, :p + 1], v[:, :p + 1], alpha[:, :p + 1],
                               None if beta is None else beta[:, :p + 1], S_in0)
        want = np.einsum("bhij,bhi->bhj", Sp, q[:, p])
        assert rel_fro(r["O"][:, i], want) <= 1e-12


def test_seam_delta_rule_retrieval():
    """alpha = beta = 1, unit keys, q_t = k_t: the state after token t maps k_t
    to v_t, so every seam output equals its value row."""
    B, H, dk, dv, NS = 1, 3, 8, 5, 6
    rng = np.random.default_rng(7)
    k = rng.standard_normal((B, NS, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, NS, H, dv))
    one = np.ones((B, NS, H))
    P = 2
    lam = np.zeros((P, B, H))
    That = np.broadcast_to(np.eye(dk), (P, B, H, dk, dk)).copy()
    Sp = rng.standard_normal((P, B, H, dk, dv))
    S_in = rng.standard_normal((1, B, H, dk, dv))
    _, O = oracle.seam_compose(DENSE, lam, That, Sp, [0, 2], [1, 0], [0, 2, NS], k, k, v, one,
                               one, S_in)
    np.testing.assert_allclose(O, v, rtol=1e-12, atol=1e-12)


def _frac_T(form, k, a, b):
    d = len(k)
    if form == KDA:  # (I - b k k^T) Diag(a): column j carries gate a_j
        return [[(Fraction(int(i == j)) - b * k[i] * k[j]) * a[j] for j in range(d)]
                for i in range(d)]
    return [[(a[0] if form != DIAG else a[i]) * (Fraction(int(i == j))
             - (b * k[i] * k[j] if form == DENSE else 0)) for j in range(d)] for i in range(d)]


def _fmat(A, B):
    return [[sum(A[i][l] * B[l][j] for l in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
@pytest.mark.parametrize("seed", [0, 1])
def test_seam_exact_rational(form, seed):
    """Exact rationals over explicit matrices: per seam token S <- T_t S + b k v^T
    and o = S^T q; per entry then S <- (e^lam That) S + S_p with lam = 0 and a
    dyadic That.  The fp64 oracle agrees to rounding."""
    rng = np.random.default_rng(300 + seed)
    dk, dv, NS, P = 3, 2, 5, 3
    dy = lambda shape: rng.integers(-8, 9, size=shape) / 8.0
    q, k, v = dy((NS, dk)), dy((NS, dk)), dy((NS, dv))
    alpha = rng.integers(1, 9, size=(NS, dk if form in (DIAG, KDA) else 1)) / 8.0
    beta = rng.integers(0, 9, size=NS) / 8.0
    That = dy((P, dk, dk))
    Sp = dy((P, dk, dv))
    S_in = dy((dk, dv))
    chain = [2, 0, 1]
    seam_off = [0, 2, 2, 5]  # entry 1 has no seam window
    if form not in (DENSE, KDA):  # scalar / diagonal pairs carry That = I
        That = np.broadcast_to(np.eye(dk), (P, dk, dk))
    F = lambda a: [[Fraction(x) for x in r] for r in np.atleast_2d(a)]
    S = F(S_in)
    O = []
    for e, p in enumerate(chain):
        for t in range(seam_off[e], seam_off[e + 1]):
            kt, vt, qt = F(k[t])[0], F(v[t])[0], F(q[t])[0]
            bt = Fraction(beta[t]) if form in (DENSE, KDA) else Fraction(1)
            TS = _fmat(_frac_T(form, kt, F(alpha[t])[0], bt), S)
            S = [[TS[i][j] + bt * kt[i] * vt[j] for j in range(dv)] for i in range(dk)]
            O.append([sum(qt[i] * S[i][j] for i in range(dk)) for j in range(dv)])
        TS = _fmat(F(That[p]), S)
        Spp = F(Sp[p])
        S = [[TS[i][j] + Spp[i][j] for j in range(dv)] for i in range(dk)]
    exact_S = np.array([[float(x) for x in r] for r in S])
    exact_O = np.array([[float(x) for x in r] for r in O])
    a_in = alpha[None, :, None, :] if form in (DIAG, KDA) else alpha[None, :, None, 0]
    That_in = That[:, None, None] if form in (DENSE, KDA) else None
    for literal in (False, True):
        S_out, O_got = oracle.seam_compose(
            form, np.zeros((P, 1, 1, dk) if form == DIAG else (P, 1, 1)), That_in,
            Sp[:, None, None], [0, 3], chain, seam_off, q[None, :, None], k[None, :, None],
            v[None, :, None], a_in, beta[None, :, None], S_in[None, None, None], literal=literal)
        scale = max(1.0, np.abs(exact_S).max())
        assert np.abs(S_out[0, 0, 0] - exact_S).max() <= 1e-13 * scale
        assert np.abs(O_got[0, :, 0] - exact_O).max() <= 1e-13 * max(1.0, np.abs(exact_O).max())


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
def test_seam_empty_windows_equal_compose(form):
    """With every window empty, reuse with seams is plain composition."""
    B, H, dk, dv, P = 2, 2, 5, 4, 4
    rng = np.random.default_rng(11)
    lam = rng.uniform(-2, 0, size=(P, B, H, dk) if form == DIAG else (P, B, H))
    That = rng.standard_normal((P, B, H, dk, dk)) * 0.3 if form in (DENSE, KDA) else None
    S = rng.standard_normal((P, B, H, dk, dv))
    S_in = rng.standard_normal((2, B, H, dk, dv))
    off, idx = [0, 3, 5], [1, 3, 0, 2, 2]
    z = np.zeros((B, 0, H, dk))
    a0 = np.zeros((B, 0, H, dk) if form in (DIAG, KDA) else (B, 0, H))
    got, O = oracle.seam_compose(form, lam, That, S, off, idx, [0] * 6, z, z,
                                 np.zeros((B, 0, H, dv)), a0, None, S_in)
    want = oracle.compose(form, lam, That, S, off, idx, S_in)
    np.testing.assert_array_equal(got, want)
    assert O.shape == (B, 0, H, dv)


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
def test_seam_queries_only_reach_outputs(form):
    """q never changes the state, and the outputs are linear in q."""
    r1 = run_split(form, [6, 7, 5], [0, 3, 2], seed=5)
    q2 = 2.0 * r1["q"] - 0.5
    seam_pos, rem_off, seam_off, rem_pos = split_prompt([6, 7, 5], [0, 3, 2])
    k, v, alpha, beta = r1["k"], r1["v"], r1["alpha"], r1["beta"]
    pool = oracle.build(form, _take(k, rem_pos), _take(v, rem_pos), _take(alpha, rem_pos),
                        _take(beta, rem_pos), rem_off)
    S2, O2 = oracle.seam_compose(form, pool["lam"], pool.get("That"), pool["S"], [0, 3],
                                 [0, 1, 2], seam_off, _take(q2, seam_pos), _take(k, seam_pos),
                                 _take(v, seam_pos), _take(alpha, seam_pos),
                                 _take(beta, seam_pos), r1["S_in"])
    np.testing.assert_array_equal(S2, r1["S_out"])
    q0 = np.zeros_like(r1["q"]) - 0.5
    _, O0 = oracle.seam_compose(form, pool["lam"], pool.get("That"), pool["S"], [0, 3],
                                [0, 1, 2], seam_off, _take(q0, seam_pos), _take(k, seam_pos),
                                _take(v, seam_pos), _take(alpha, seam_pos),
                                _take(beta, seam_pos), r1["S_in"])
    np.testing.assert_allclose(O2, 2.0 * r1["O"] + O0, rtol=1e-11, atol=1e-11)


def test_seam_oracle_rejects_bad_seam_offsets():
    P, B, H, dk, dv = 2, 1, 1, 4, 4
    lam = np.zeros((P, B, H))
    S = np.zeros((P, B, H, dk, dv))
    x = np.zeros((B, 3, H, dk))
    a = np.ones((B, 3, H))
    for bad in ([1, 2, 3], [0, 2, 1], [0, 1, 2]):
        with pytest.raises(ValueError):
            oracle.seam_compose(SCALAR, lam, None, S, [0, 2], [0, 1], bad, x, x,
                                np.zeros((B, 3, H, dv)), a, None)


def test_seam_kda_with_shared_gates_is_the_dense_seam():
    """Every channel of a token sharing one gate: the KDA seam step is the
    dense one ((I - b k k^T) a = a (I - b k k^T)), so state and outputs agree."""
    seg_lens, seam_lens = [7, 9, 5], [0, 3, 3]
    B, H, dk, dv = 2, 2, 6, 5
    N = sum(seg_lens)
    q, k, v, a1, beta = _inputs(DENSE, B, H, dk, dv, N, seed=21)
    a_all = np.repeat(a1[..., None], dk, axis=-1)
    seam_pos, rem_off, seam_off, rem_pos = split_prompt(seg_lens, seam_lens)
    pool_d = oracle.build(DENSE, _take(k, rem_pos), _take(v, rem_pos), _take(a1, rem_pos),
                          _take(beta, rem_pos), rem_off)
    pool_k = oracle.build(KDA, _take(k, rem_pos), _take(v, rem_pos), _take(a_all, rem_pos),
                          _take(beta, rem_pos), rem_off)
    S_in = np.random.default_rng(22).standard_normal((1, B, H, dk, dv))
    args = lambda a: (seam_off, _take(q, seam_pos), _take(k, seam_pos), _take(v, seam_pos),
                      _take(a, seam_pos), _take(beta, seam_pos), S_in)
    Sd, Od = oracle.seam_compose(DENSE, pool_d["lam"], pool_d["That"], pool_d["S"], [0, 3],
                                 [0, 1, 2], *args(a1))
    Sk, Ok = oracle.seam_compose(KDA, pool_k["lam"], pool_k["That"], pool_k["S"], [0, 3],
                                 [0, 1, 2], *args(a_all))
    assert rel_fro(Sk, Sd) <= 1e-12
    assert rel_fro(Ok, Od) <= 1e-12
