"""Pins of the oracle's re-rotation of cached pairs (rotary position
embeddings on the keys).  [xix.ai HYPIC article (French), paragraph on linear
layers: variants with rotary embeddings need the cached state re-rotated.]

Reading: a segment built with its keys rotated at positions 0..L-1 and placed
at offset p has every key rotated by R_p on top, so its pair becomes
(lambda, R_p That R_p^T, R_p S).  The pins check this against the oracle's
build run on keys rotated with complex arithmetic (not with the oracle's
matrix), the angles against hand values, and the rotation's group law,
orthogonality and the relation between the two channel pairings.
"""
import numpy as np
import pytest

import oracle
from oracle import DENSE, DIAG, KDA, ROPE_HALF, ROPE_INTERLEAVED, SCALAR
from tests.conftest import rel_fro


def rope_keys(k, positions, rot_dim, base, pairing):
    """Rotary embedding of keys k [..., N, H, dk] at the given positions (one
    per token), as multiplication of complex numbers x_a + i x_b by
    exp(i * pos * base^(-2j/rot_dim))."""
    k = np.array(k, dtype=np.float64)
    h = rot_dim // 2
    if pairing == ROPE_INTERLEAVED:
        a_idx, b_idx = np.arange(0, rot_dim, 2), np.arange(1, rot_dim, 2)
    else:
        a_idx, b_idx = np.arange(h), np.arange(h, rot_dim)
    z = k[..., a_idx] + 1j * k[..., b_idx]
    freq = base ** (-2.0 * np.arange(h) / rot_dim)
    pos = np.asarray(positions, dtype=np.float64)
    rot = np.exp(1j * pos[:, None, None] * freq[None, None, :])     # [N, 1, h]
    z = z * rot
    out = k.copy()
    out[..., a_idx] = z.real
    out[..., b_idx] = z.imag
    return out


def inputs(form, B, H, dk, dv, N, seed, pair_gates=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, H, dv))
    if form in (DIAG, KDA):
        a = rng.uniform(0.6, 1.0, size=(B, N, H, dk))
        if pair_gates:  # the two channels of every interleaved pair share a gate
            a[..., 1::2] = a[..., 0::2]
    else:
        a = rng.uniform(0.6, 1.0, size=(B, N, H))
    b = rng.uniform(0.0, 1.0, size=(B, N, H))
    return k, v, a, b


CASES = [(SCALAR, ROPE_INTERLEAVED, 8), (DENSE, ROPE_INTERLEAVED, 8), (DENSE, ROPE_HALF, 8),
         (DENSE, ROPE_HALF, 4), (DIAG, ROPE_INTERLEAVED, 8), (KDA, ROPE_INTERLEAVED, 6)]


@pytest.mark.parametrize("form,pairing,rot_dim", CASES)
def test_rerotated_pair_is_the_pair_at_the_new_position(form, pairing, rot_dim):
    dk, dv, L = 8, 5, 23
    k, v, a, b = inputs(form, 1, 2, dk, dv, L, seed=10 + form)
    base = 10000.0
    offs = [0, L]
    rel = rope_keys(k, np.arange(L), rot_dim, base, pairing)
    for p in (0, 1, 37, 4095, 131071):
        absk = rope_keys(k, p + np.arange(L), rot_dim, base, pairing)
        built = oracle.build(form, rel, v, a, b, offs)
        want = oracle.build(form, absk, v, a, b, offs)
        lam, That, S = oracle.rerotate(form, built["lam"], built.get("That"), built["S"], [0], [p],
                                       rot_dim, base, pairing)
        assert rel_fro(S, want["S"]) <= 1e-11, p
        assert np.array_equal(lam, want["lam"])
        if form in (DENSE, KDA):
            assert rel_fro(That, want["That"]) <= 1e-11, p


def test_unequal_gates_in_a_pair_do_not_rerotate():
    """The reading's condition: with per-channel gates that differ within a
    rotated pair, the rotated pair is not the pair at the new position."""
    dk, dv, L = 8, 4, 20
    for form in (DIAG, KDA):
        k, v, a, b = inputs(form, 1, 1, dk, dv, L, seed=3, pair_gates=False)
        rel = rope_keys(k, np.arange(L), dk, 100.0, ROPE_INTERLEAVED)
        absk = rope_keys(k, 50 + np.arange(L), dk, 100.0, ROPE_INTERLEAVED)
        built = oracle.build(form, rel, v, a, b, [0, L])
        want = oracle.build(form, absk, v, a, b, [0, L])
        _, _, S = oracle.rerotate(form, built["lam"], built.get("That"), built["S"], [0], [50], dk,
                                  100.0)
        assert rel_fro(S, want["S"]) > 1e-3


def test_rope_matrix_hand_values():
    """rot_dim 4, base 100: pair 0 turns by p radians, pair 1 by p/10."""
    for p in (1, 3):
        R = oracle.rope_matrix(5, p, 4, 100.0, ROPE_INTERLEAVED)
        c0, s0, c1, s1 = np.cos(p), np.sin(p), np.cos(p / 10), np.sin(p / 10)
        want = np.array([[c0, -s0, 0, 0, 0], [s0, c0, 0, 0, 0], [0, 0, c1, -s1, 0],
                         [0, 0, s1, c1, 0], [0, 0, 0, 0, 1]])
        assert np.abs(R - want).max() <= 1e-15
        H = oracle.rope_matrix(5, p, 4, 100.0, ROPE_HALF)
        want_h = np.array([[c0, 0, -s0, 0, 0], [0, c1, 0, -s1, 0], [s0, 0, c0, 0, 0],
                           [0, s1, 0, c1, 0], [0, 0, 0, 0, 1]])
        assert np.abs(H - want_h).max() <= 1e-15


@pytest.mark.parametrize("pairing", [ROPE_INTERLEAVED, ROPE_HALF])
def test_group_law_orthogonality_and_identity(pairing):
    dk, rot = 16, 12
    for p, q in ((3, 5), (1000, -1000), (65536, 12345)):
        Rp = oracle.rope_matrix(dk, p, rot, 10000.0, pairing)
        Rq = oracle.rope_matrix(dk, q, rot, 10000.0, pairing)
        Rpq = oracle.rope_matrix(dk, p + q, rot, 10000.0, pairing)
        assert np.abs(Rp @ Rq - Rpq).max() <= 1e-10
        assert np.abs(Rp @ Rp.T - np.eye(dk)).max() <= 1e-14
    assert np.array_equal(oracle.rope_matrix(dk, 0, rot, 10000.0, pairing), np.eye(dk))
    rng = np.random.default_rng(0)
    S = rng.standard_normal((3, 1, 2, dk, 4))
    T = rng.standard_normal((3, 1, 2, dk, dk))
    lam = rng.standard_normal((3, 1, 2))
    l0, T0, S0 = oracle.rerotate(DENSE, lam, T, S, [2, 0], [0, 0], rot, 10000.0, pairing)
    assert np.array_equal(S0, S[[2, 0]]) and np.array_equal(T0, T[[2, 0]])
    _, T1, S1 = oracle.rerotate(DENSE, lam, T, S, [1], [777], rot, 10000.0, pairing)
    assert abs(np.linalg.norm(S1) - np.linalg.norm(S[1])) <= 1e-12 * np.linalg.norm(S[1])
    assert abs(np.linalg.norm(T1) - np.linalg.norm(T[1])) <= 1e-12 * np.linalg.norm(T[1])
    # channels at and past rot_dim are left alone
    assert np.array_equal(S1[0, ..., rot:, :], S[1, ..., rot:, :])


def test_half_pairing_is_a_permuted_interleaving():
    """R_half = P R_interleaved P^T, P sending channel 2i to i and 2i+1 to
    i + rot/2 (channels past rot_dim fixed)."""
    dk, rot = 10, 8
    perm = list(range(0, rot, 2)) + list(range(1, rot, 2)) + list(range(rot, dk))
    P = np.zeros((dk, dk))
    for new, old in enumerate(perm):
        P[new, old] = 1.0
    for p in (1, 99):
        Ri = oracle.rope_matrix(dk, p, rot, 500.0, ROPE_INTERLEAVED)
        Rh = oracle.rope_matrix(dk, p, rot, 500.0, ROPE_HALF)
        assert np.abs(P @ Ri @ P.T - Rh).max() <= 1e-15


@pytest.mark.parametrize("form", [SCALAR, DENSE])
def test_segments_built_at_zero_moved_and_composed_equal_the_prompt(form):
    """The use on reuse: segments built at relative positions, moved to their
    offsets in the prompt and composed, give the recurrence over the prompt's
    keys rotated at absolute positions."""
    dk, dv = 8, 6
    cuts = [0, 17, 17, 40, 71]
    N = cuts[-1]
    k, v, a, b = inputs(form, 1, 2, dk, dv, N, seed=21)
    base, rot = 10000.0, 8
    rel = np.concatenate([rope_keys(k[:, cuts[s]:cuts[s + 1]], np.arange(cuts[s + 1] - cuts[s]),
                                    rot, base, ROPE_HALF) for s in range(len(cuts) - 1)], axis=1)
    built = oracle.build(form, rel, v, a, b, cuts)
    n = len(cuts) - 1
    lam, That, S = oracle.rerotate(form, built["lam"], built.get("That"), built["S"], list(range(n)),
                                   cuts[:-1], rot, base, ROPE_HALF)
    got = oracle.compose(form, lam, That, S, [0, n], list(range(n)))
    absk = rope_keys(k, np.arange(N), rot, base, ROPE_HALF)
    want = oracle.recurrence(form, absk, v, a, b)
    assert rel_fro(got[0], want) <= 1e-11


def _mutant_rope(kind):
    """rope_matrix with one planted mistake."""
    def R(dk, shift, rot_dim, base, pairing=ROPE_INTERLEAVED):
        M = np.eye(dk)
        h = rot_dim // 2
        for i in range(h):
            a, b = (2 * i, 2 * i + 1) if pairing == ROPE_INTERLEAVED else (i, i + h)
            if kind == "pairing swapped":
                a, b = (i, i + h) if pairing == ROPE_INTERLEAVED else (2 * i, 2 * i + 1)
            expo = -1.0 * i / rot_dim if kind == "exponent -i/d" else -2.0 * i / rot_dim
            phi = float(shift) * float(base) ** expo
            c, s = np.cos(phi), np.sin(phi)
            if kind == "transposed":
                s = -s
            M[a, a], M[a, b], M[b, a], M[b, b] = c, -s, s, c
            if kind == "last pair skipped" and i == h - 1:
                M[a, a], M[a, b], M[b, a], M[b, b] = 1.0, 0.0, 0.0, 1.0
        return M
    return R


@pytest.mark.parametrize("kind", ["pairing swapped", "exponent -i/d", "transposed",
                                  "last pair skipped"])
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(oracle, "rope_matrix", _mutant_rope(kind))
    checks = [lambda: test_rerotated_pair_is_the_pair_at_the_new_position(DENSE, ROPE_HALF, 8),
              lambda: test_rerotated_pair_is_the_pair_at_the_new_position(DENSE,
                                                                          ROPE_INTERLEAVED, 8),
              test_rope_matrix_hand_values]
    caught = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught > 0, kind
