"""Parity of the HIP re-rotation of cached pairs (rotary embeddings on the
keys) with the fp64 oracle, through the C ABI: every form, both channel
pairings, partial rotary dimensions, zero / negative / very long shifts,
repeated pool entries; and its use on reuse -- segments built on the GPU at
relative positions, moved to their offsets and composed -- against the
oracle's recurrence over the prompt's keys rotated at absolute positions.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import DENSE, DIAG, KDA, ROPE_HALF, ROPE_INTERLEAVED, SCALAR
from tests.gpu_helpers import TOL_BF16, TOL_F32, max_rel_units, report, to_dev
from tests.test_oracle_rope_pins import rope_keys

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def random_pool(form, P, B, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    lam = rng.standard_normal((P, B, H, dk) if form == DIAG else (P, B, H)).astype(np.float32)
    T = rng.standard_normal((P, B, H, dk, dk)).astype(np.float32) if form in (DENSE, KDA) else None
    S = rng.standard_normal((P, B, H, dk, dv)).astype(np.float32)
    return lam, T, S


CASES = [(DENSE, 128, 128, 128, ROPE_HALF), (DENSE, 128, 128, 64, ROPE_INTERLEAVED),
         (KDA, 64, 96, 64, ROPE_HALF), (SCALAR, 128, 64, 32, ROPE_INTERLEAVED),
         (DIAG, 32, 48, 16, ROPE_HALF), (DENSE, 16, 16, 8, ROPE_INTERLEAVED),
         (DENSE, 96, 32, 96, ROPE_HALF)]


@pytest.mark.parametrize("form,dk,dv,rot,pairing", CASES)
def test_rerotate_matches_oracle(form, dk, dv, rot, pairing):
    import hybrid_caching_amd as pic
    import torch
    P, B, H = 4, 2, 3
    lam, T, S = random_pool(form, P, B, H, dk, dv, seed=dk + rot + form)
    idx = [3, 0, 0, 2, 1, 3]
    shift = [0, 1, -1, 4096, 1_000_003, -77777]
    base = 10000.0
    out = pic.pic_rerotate(form, to_dev(lam), to_dev(T), to_dev(S), idx, shift, rot, base,
                           pairing)
    torch.cuda.synchronize()
    l_ref, T_ref, S_ref = oracle.rerotate(form, lam, T, S, idx, shift, rot, base, pairing)
    assert np.array_equal(out["log_scale"].cpu().numpy(), l_ref.astype(np.float32))
    e_s = max_rel_units(out["S0"].cpu().numpy(), S_ref)
    msg = f"S0 err {e_s:.3e}"
    e_t = 0.0
    if T is not None:
        e_t = max_rel_units(out["T_hat"].cpu().numpy(), T_ref)
        msg += f", That err {e_t:.3e}"
    report(msg)
    assert e_s <= TOL_F32 and e_t <= TOL_F32, msg
    # shift 0 is a copy, bit for bit
    assert np.array_equal(out["S0"][0].cpu().numpy(), S[3])
    if T is not None:
        assert np.array_equal(out["T_hat"][0].cpu().numpy(), T[3])


def test_rerotate_nothing_to_do():
    import hybrid_caching_amd as pic
    import torch
    lam, T, S = random_pool(DENSE, 2, 1, 1, 32, 32, seed=1)
    out = pic.pic_rerotate(DENSE, to_dev(lam), to_dev(T), to_dev(S), [], [], 32)
    torch.cuda.synchronize()
    assert out["S0"].shape[0] == 0


@pytest.mark.parametrize("form", [DENSE, SCALAR, KDA])
def test_moved_segments_compose_into_the_prompt(form):
    """Segments built on the GPU with keys rotated at positions relative to
    each segment, moved to their offsets, composed: the oracle's recurrence
    over the same keys rotated at absolute positions.  KDA gates are shared
    within each rotated channel pair (the condition of the reading)."""
    import hybrid_caching_amd as pic
    import torch
    B, H, dk, dv = 2, 2, 128, 64
    cuts = [0, 200, 200, 333, 700]
    N = cuts[-1]
    rng = np.random.default_rng(5 + form)
    k = rng.standard_normal((B, N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, H, dv)).astype(np.float32)
    rot, base = 64, 10000.0
    if form == KDA:
        a = rng.uniform(0.995, 1.0, size=(B, N, H, dk)).astype(np.float32)
        a[..., rot // 2:rot] = a[..., :rot // 2]  # half pairing: channel i pairs with i + rot/2
    else:
        a = rng.uniform(0.995, 1.0, size=(B, N, H)).astype(np.float32)
    b = rng.uniform(0.0, 0.05, size=(B, N, H)).astype(np.float32) if form != SCALAR else None
    n = len(cuts) - 1
    rel = np.concatenate([rope_keys(k[:, cuts[s]:cuts[s + 1]], np.arange(cuts[s + 1] - cuts[s]),
                                    rot, base, ROPE_HALF) for s in range(n)], axis=1)
    rel = rel.astype(np.float32)
    dt = torch.float32
    pair = pic.pic_segment_build(form, to_dev(rel, dt), to_dev(v, dt), to_dev(a), to_dev(b), cuts)
    moved = pic.pic_rerotate(form, pair["log_scale"], pair.get("T_hat"), pair["S0"],
                             list(range(n)), cuts[:-1], rot, base, ROPE_HALF)
    S_in = synth.random_state((1, B, H, dk, dv), seed=9)
    got = pic.pic_compose(form, moved["log_scale"], moved.get("T_hat"), moved["S0"], [0, n],
                          list(range(n)), to_dev(S_in))
    torch.cuda.synchronize()
    absk = rope_keys(k, np.arange(N), rot, base, ROPE_HALF).astype(np.float32)
    want = oracle.recurrence(form, absk, v, a, b, S_in[0])
    e = max_rel_units(got.cpu().numpy()[0], want)
    # not moving the pairs is visibly wrong
    unmoved = pic.pic_compose(form, pair["log_scale"], pair.get("T_hat"), pair["S0"], [0, n],
                              list(range(n)), to_dev(S_in))
    torch.cuda.synchronize()
    e_un = max_rel_units(unmoved.cpu().numpy()[0], want)
    report(f"form {form}: moved and composed err {e:.3e}; without moving {e_un:.3e}")
    assert e <= TOL_F32
    assert e_un > 1e-2


def test_rerotate_rejects_overlap_and_leaves_outputs():
    import hybrid_caching_amd as pic
    import torch
    lam, T, S = random_pool(DENSE, 2, 1, 1, 32, 32, seed=2)
    dl, dT, dS = to_dev(lam), to_dev(T), to_dev(S)
    with pytest.raises(pic.PicError):
        pic.pic_rerotate(DENSE, dl, dT, dS, [0], [5], 32, out={"log_scale": dl[1:], "T_hat": dT[1:],
                                                                "S0": dS[1:]})
    torch.cuda.synchronize()
    assert np.array_equal(dS.cpu().numpy(), S) and np.array_equal(dT.cpu().numpy(), T)
