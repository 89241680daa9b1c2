"""Parity of reuse with seam windows (``pic_compose_seams``) with the fp64
oracle, through the C ABI: every chain entry first runs its seam tokens from
the running state, each writing o_t = S_t^T q_t, then applies its pair.
[xix.ai HYPIC article (French), paragraph on full-attention layers: seam
windows of w tokens (8 by default) recomputed on reuse; the linear layers
advance the running state through them and pass each token's output up.]

The seam updates and the state are fp32 on the GPU; bf16 inputs are exact on
both sides (the oracle reads the same rounded values), so the fp32 contract
tolerance applies to states and outputs alike, except where a bf16 build is
part of the path.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import DENSE, DIAG, KDA, SCALAR
from tests.gpu_helpers import TOL_BF16, TOL_F32, max_rel_units, report, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()  # fails loudly if the HIP library is missing


def random_pool(form, P, B, H, dk, dv, seed, lam_range=(-1.0, 0.0)):
    rng = np.random.default_rng(seed)
    lam = rng.uniform(*lam_range, size=(P, B, H, dk) if form == DIAG else (P, B, H)).astype(np.float32)
    That = None
    if form in (DENSE, KDA):
        That = np.empty((P, B, H, dk, dk), dtype=np.float32)
        for idx in np.ndindex(P, B, H):
            M = np.eye(dk)
            for _ in range(3):
                x = rng.standard_normal(dk)
                x /= np.linalg.norm(x)
                M = (np.eye(dk) - rng.uniform(0, 1) * np.outer(x, x)) @ M
            That[idx] = M
    S = (0.3 * rng.standard_normal((P, B, H, dk, dv))).astype(np.float32)
    return lam, That, S


def seam_inputs(form, B, NS, H, dk, dv, seed, bf16, alpha=(0.9, 1.0), unit_keys=True):
    """Seam tokens with the build workloads' distributions, rounded to the
    storage type: keys L2-normalised (dense) or 1/sqrt(dk)-scaled."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, NS, H, dk)).astype(np.float32)
    if form in (DENSE, KDA) and unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k *= np.float32(1 / np.sqrt(dk))
    q = (rng.standard_normal((B, NS, H, dk)) / np.sqrt(dk)).astype(np.float32)
    v = rng.standard_normal((B, NS, H, dv)).astype(np.float32)
    if bf16:
        q, k, v = synth.bf16_round(q), synth.bf16_round(k), synth.bf16_round(v)
    if form in (DIAG, KDA):
        a = (1 / (1 + np.exp(-rng.normal(3.0, 1.0, size=(B, NS, H, dk))))).astype(np.float32)
    else:
        a = rng.uniform(*alpha, size=(B, NS, H)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, size=(B, NS, H)).astype(np.float32) if form in (DENSE, KDA) else None
    return q, k, v, a, b


def run_both(form, lam, That, S, off, idx, seam_off, q, k, v, a, b, S_in, bf16):
    import hybrid_caching_amd as pic
    import torch
    dt = torch.bfloat16 if bf16 else torch.float32
    S_out, O = pic.pic_compose_seams(form, to_dev(lam), to_dev(That), to_dev(S), off, idx,
                                     seam_off, to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                                     to_dev(a), to_dev(b), to_dev(S_in))
    torch.cuda.synchronize()
    ref_S, ref_O = oracle.seam_compose(form, lam, That, S, off, idx, seam_off, q, k, v, a, b, S_in)
    return S_out.cpu().numpy(), O.cpu().numpy(), ref_S, ref_O


def out_err(O, ref_O):
    """Max over (layer, head) of the relative Frobenius error of all outputs."""
    return max_rel_units(np.moveaxis(O, 1, 2), np.moveaxis(ref_O, 1, 2))


CHAINS = ([0, 5, 5, 12, 13], [3, 0, 7, 7, 1, 2, 3, 4, 5, 6, 8, 9, 0])
WINDOWS = [0, 8, 3, 8, 0, 1, 8, 8, 5, 16, 64, 8, 2]  # per chain entry


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("bf16", [True, False])
def test_seam_compose_matches_oracle(form, d, bf16):
    P, B, H = 10, 2, 3
    lam, That, S = random_pool(form, P, B, H, d, d, seed=40 + d + form)
    off, idx = CHAINS
    seam_off = np.concatenate([[0], np.cumsum(WINDOWS)])
    NS = int(seam_off[-1])
    q, k, v, a, b = seam_inputs(form, B, NS, H, d, d, seed=60 + d + form, bf16=bf16)
    S_in = synth.random_state((len(off) - 1, B, H, d, d), seed=5, scale=0.5)
    got_S, got_O, ref_S, ref_O = run_both(form, lam, That, S, off, idx, seam_off, q, k, v, a, b,
                                          S_in, bf16)
    es, eo = max_rel_units(got_S, ref_S), out_err(got_O, ref_O)
    report(f"seam compose state err {es:.3e}, output err {eo:.3e}")
    assert es <= TOL_F32 and eo <= TOL_F32


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (32, 96)])
def test_seam_compose_unequal_dims(dk, dv):
    P, B, H = 6, 1, 2
    lam, That, S = random_pool(DENSE, P, B, H, dk, dv, seed=dk + dv)
    off, idx = [0, 4, 7], [5, 1, 0, 2, 3, 3, 4]
    seam_off = np.concatenate([[0], np.cumsum([0, 8, 8, 4, 8, 1, 8])])
    NS = int(seam_off[-1])
    q, k, v, a, b = seam_inputs(DENSE, B, NS, H, dk, dv, seed=dk * dv, bf16=True)
    S_in = synth.random_state((2, B, H, dk, dv), seed=9, scale=0.5)
    got_S, got_O, ref_S, ref_O = run_both(DENSE, lam, That, S, off, idx, seam_off, q, k, v, a, b,
                                          S_in, True)
    assert max_rel_units(got_S, ref_S) <= TOL_F32
    assert out_err(got_O, ref_O) <= TOL_F32


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
def test_seam_windows_empty_equal_compose(form):
    """With every window empty the call is a plain compose.  The dense
    kernels multiply by e^lambda on different sides of the split-bf16 product
    (each product is exact to about 2^-16 relative), so the dense form agrees
    to a few 1e-6 rather than to the last bit; each is pinned against the
    oracle on its own."""
    import hybrid_caching_amd as pic
    import torch
    P, B, H, d = 10, 2, 3, 128
    lam, That, S = random_pool(form, P, B, H, d, d, seed=11 + form)
    off, idx = CHAINS
    S_in = synth.random_state((len(off) - 1, B, H, d, d), seed=6)
    z = torch.zeros((B, 0, H, d), dtype=torch.float32, device="cuda")
    za = torch.zeros((B, 0, H, d) if form in (DIAG, KDA) else (B, 0, H), dtype=torch.float32,
                     device="cuda")
    got, O = pic.pic_compose_seams(form, to_dev(lam), to_dev(That), to_dev(S), off, idx,
                                   [0] * (len(idx) + 1), z, z, z, za, None, to_dev(S_in))
    want = pic.pic_compose(form, to_dev(lam), to_dev(That), to_dev(S), off, idx, to_dev(S_in))
    torch.cuda.synchronize()
    assert O.shape == (B, 0, H, d)
    assert max_rel_units(got.cpu().numpy(), want.cpu().numpy()) <= (3e-5 if form in (DENSE, KDA)
                                                                    else 1e-6)


def test_seam_delta_rule_retrieval():
    """alpha = beta = 1, unit keys, q_t = k_t: each output equals its value."""
    P, B, H, d = 3, 1, 4, 128
    lam = np.zeros((P, B, H), dtype=np.float32)
    That = np.broadcast_to(np.eye(d, dtype=np.float32), (P, B, H, d, d)).copy()
    rng = np.random.default_rng(17)
    S = (0.3 * rng.standard_normal((P, B, H, d, d))).astype(np.float32)
    off, idx = [0, 3], [2, 0, 1]
    seam_off = [0, 8, 16, 24]
    _, k, v, _, _ = seam_inputs(DENSE, B, 24, H, d, d, seed=18, bf16=False)
    one = np.ones((B, 24, H), dtype=np.float32)
    got_S, got_O, ref_S, ref_O = run_both(DENSE, lam, That, S, off, idx, seam_off, k, k, v, one,
                                          one, None, False)
    e = float(np.max(np.abs(got_O - v)))
    report(f"seam retrieval max |o - v| {e:.3e}")
    assert e <= 1e-4 * max(1.0, float(np.max(np.abs(v))))
    # the keys are normalised in fp32, so |k|^2 = 1 holds to ~1e-7 only
    assert np.max(np.abs(ref_O - v)) <= 1e-5


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
@pytest.mark.parametrize("n_req,steps", [(16, 4), (17, 3), (4, 40)])
def test_seam_tables_in_arguments_and_in_workspace(form, n_req, steps):
    """Chain and seam tables travel in the kernel arguments up to 16 requests
    and 64 entries, and through the workspace beyond."""
    P, B, H, d = 12, 1, 2, 64
    lam, That, S = random_pool(form, P, B, H, d, d, seed=70 + n_req + steps)
    rng = np.random.default_rng(n_req * 100 + steps)
    off = np.arange(n_req + 1) * steps
    idx = rng.integers(0, P, size=off[-1]).astype(np.int32)
    w = rng.integers(0, 9, size=off[-1])
    seam_off = np.concatenate([[0], np.cumsum(w)])
    q, k, v, a, b = seam_inputs(form, B, int(seam_off[-1]), H, d, d, seed=3, bf16=True)
    got_S, got_O, ref_S, ref_O = run_both(form, lam, That, S, off, idx, seam_off, q, k, v, a, b,
                                          None, True)
    assert max_rel_units(got_S, ref_S) <= TOL_F32
    assert out_err(got_O, ref_O) <= TOL_F32


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE, KDA])
def test_seam_split_equals_unsplit_slow_gates(form):
    """End to end: a prompt of segments whose inner segments start with an
    8-token seam window; the windows' remainders are built on the GPU, then
    reused with their seams from S = 0.  The final state matches the unsplit
    recurrence over the whole prompt, and every seam output matches the
    oracle's (slow gates, so the carried state is a sizeable part)."""
    import hybrid_caching_amd as pic
    import torch
    B, H, d = 1, 4, 128
    seg_lens, w = [300, 129, 400, 195], 8
    N = sum(seg_lens)
    rng = np.random.default_rng(900 + form)
    k = rng.standard_normal((B, N, H, d)).astype(np.float32)
    erase = form in (DENSE, KDA)
    if erase:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k *= np.float32(1 / np.sqrt(d))
    q = (rng.standard_normal((B, N, H, d)) / np.sqrt(d)).astype(np.float32)
    v = rng.standard_normal((B, N, H, d)).astype(np.float32)
    if not erase:
        v *= np.float32(1 / np.sqrt(d))
    q, k, v = synth.bf16_round(q), synth.bf16_round(k), synth.bf16_round(v)
    a = rng.uniform(0.999, 1.0, size=(B, N, H, d) if form in (DIAG, KDA) else (B, N, H)).astype(np.float32)
    b = rng.uniform(0.0, 0.05, size=(B, N, H)).astype(np.float32) if erase else None
    seam_pos, rem_pos, seam_off, rem_off, start = [], [], [0], [0], 0
    for i, L in enumerate(seg_lens):
        wi = w if i > 0 else 0
        seam_pos += range(start, start + wi)
        rem_pos += range(start + wi, start + L)
        seam_off.append(len(seam_pos))
        rem_off.append(len(rem_pos))
        start += L
    take = lambda x, p: None if x is None else np.ascontiguousarray(x[:, p])
    dt = torch.bfloat16
    pair = pic.pic_segment_build(form, to_dev(take(k, rem_pos), dt), to_dev(take(v, rem_pos), dt),
                                 to_dev(take(a, rem_pos)), to_dev(take(b, rem_pos)), rem_off)
    n = len(seg_lens)
    S_out, O = pic.pic_compose_seams(form, pair["log_scale"], pair.get("T_hat"), pair["S0"],
                                     [0, n], list(range(n)), seam_off,
                                     to_dev(take(q, seam_pos), dt), to_dev(take(k, seam_pos), dt),
                                     to_dev(take(v, seam_pos), dt), to_dev(take(a, seam_pos)),
                                     to_dev(take(b, seam_pos)))
    torch.cuda.synchronize()
    unsplit = oracle.recurrence(form, k, v, a, b)
    last = oracle.build(form, take(k, rem_pos), take(v, rem_pos), take(a, rem_pos),
                        take(b, rem_pos), rem_off)["S"][-1]
    rho = float(np.min(np.linalg.norm((unsplit - last).reshape(H, -1), axis=1)
                       / np.linalg.norm(unsplit.reshape(H, -1), axis=1)))
    assert rho >= 0.1, rho
    es = max_rel_units(S_out.cpu().numpy()[0], unsplit)
    pool = oracle.build(form, take(k, rem_pos), take(v, rem_pos), take(a, rem_pos),
                        take(b, rem_pos), rem_off)
    _, ref_O = oracle.seam_compose(form, pool["lam"], pool.get("That"), pool["S"], [0, n],
                                   list(range(n)), seam_off, take(q, seam_pos),
                                   take(k, seam_pos), take(v, seam_pos), take(a, seam_pos),
                                   take(b, seam_pos))
    eo = out_err(O.cpu().numpy(), ref_O)
    report(f"seam split/compose vs unsplit err {es:.3e}, outputs {eo:.3e}, rho {rho:.2f}")
    assert es <= TOL_BF16 and eo <= TOL_BF16


def test_seam_errors_leave_outputs_untouched():
    import hybrid_caching_amd as pic
    import torch
    P, B, H, d = 4, 1, 2, 32
    lam, That, S = random_pool(DENSE, P, B, H, d, d, seed=1)
    q, k, v, a, b = seam_inputs(DENSE, B, 70, H, d, d, seed=2, bf16=True)
    out = torch.full((1, B, H, d, d), 7.0, device="cuda")
    out_O = torch.full((B, 70, H, d), 7.0, device="cuda")
    dt = torch.bfloat16
    with pytest.raises(pic.PicError) as ei:  # a 65-token window
        pic.pic_compose_seams(DENSE, to_dev(lam), to_dev(That), to_dev(S), [0, 2], [0, 1],
                              [0, 5, 70], to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(a),
                              to_dev(b), out=out, out_O=out_O)
    assert ei.value.code == -2
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((out_O == 7.0).all())
