"""Parity of the HIP path with the fp64 oracle, through the C ABI (via the
ctypes binding), on seeded inputs: element by element at sizes the oracle
finishes in seconds (several chunks, ragged tails, empty segments, every
supported head size), bitwise on exact-arithmetic cases, and the error paths.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import DENSE, DIAG, SCALAR
from tests.gpu_helpers import (TOL_BF16, TOL_F32, assert_pair_close, build_both, lam_err,
                               max_rel_units, report, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()  # fails loudly if the HIP library is missing


def rand_case(form, B, H, dk, dv, offsets, seed, bf16=True, alpha=(0.9, 1.0), beta=(0.0, 1.0)):
    """Seeded inputs with the configs' distributions (k rows L2-normalised for
    the dense form, 1/sqrt(dk)-scaled otherwise), rounded to the storage type."""
    rng = np.random.default_rng(seed)
    N = int(offsets[-1])
    k = rng.standard_normal((B, N, H, dk)).astype(np.float32)
    if form == DENSE:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k *= np.float32(1 / np.sqrt(dk))
    v = rng.standard_normal((B, N, H, dv)).astype(np.float32)
    if form != DENSE:
        v *= np.float32(1 / np.sqrt(dk))
    if bf16:
        k, v = synth.bf16_round(k), synth.bf16_round(v)
    ashape = (B, N, H, dk) if form == DIAG else (B, N, H)
    if form == DIAG:
        a = (1 / (1 + np.exp(-rng.normal(3.0, 1.0, size=ashape)))).astype(np.float32)
    else:
        a = rng.uniform(*alpha, size=ashape).astype(np.float32)
    b = rng.uniform(*beta, size=(B, N, H)).astype(np.float32) if form == DENSE else None
    return k, v, a, b


RAGGED = [0, 63, 127, 127, 300, 364]  # tails of 63 / 64 / 1 tokens, an empty segment


# --------------------------------------------------------------------------
# build
# --------------------------------------------------------------------------

def test_tiny_dense_fp32_config():
    """1 layer, 2 heads, d = 16, 2 x 64 tokens, fp32: build, compose, naive add,
    compared with the oracle and with the unsplit recurrence."""
    w = synth.WORKLOADS["tiny_dense"]
    x = synth.layer_inputs(w)
    gpu, ref = build_both(DENSE, x["k"], x["v"], x["alpha"], x["beta"], x["offsets"], False)
    assert_pair_close(gpu, ref, DENSE, TOL_F32)
    import hybrid_caching_amd as pic
    import torch
    S_in = synth.random_state((1, 1, w.heads, w.dk, w.dv), seed=7)
    for sin in (None, S_in):
        out = pic.pic_compose(DENSE, to_dev(gpu["log_scale"]), to_dev(gpu["T_hat"]),
                              to_dev(gpu["S0"]), [0, 2], [0, 1], to_dev(sin))
        unsplit = oracle.recurrence(DENSE, x["k"], x["v"], x["alpha"], x["beta"],
                                    None if sin is None else sin[0])
        assert max_rel_units(out.cpu().numpy()[0], unsplit) <= TOL_F32
        nv = pic.pic_naive_add(to_dev(gpu["S0"]), [0, 2], [0, 1], to_dev(sin))
        ref_nv = oracle.naive_add(ref["S"], [0, 2], [0, 1], sin)
        assert max_rel_units(nv.cpu().numpy(), ref_nv) <= TOL_F32
    T = pic.pic_materialize_T(DENSE, to_dev(gpu["log_scale"]), to_dev(gpu["T_hat"]))
    ref_T = oracle.build(DENSE, x["k"], x["v"], x["alpha"], x["beta"], x["offsets"],
                         want_T=True)["T"]
    torch.cuda.synchronize()
    assert max_rel_units(T.cpu().numpy(), ref_T) <= TOL_F32


@pytest.mark.parametrize("d", [16, 32, 48, 64, 96, 128])
def test_dense_build_head_sizes(d):
    k, v, a, b = rand_case(DENSE, 2, 3, d, d, RAGGED, seed=100 + d)
    gpu, ref = build_both(DENSE, k, v, a, b, RAGGED, True)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (32, 96)])
def test_dense_build_unequal_dims(dk, dv):
    k, v, a, b = rand_case(DENSE, 1, 2, dk, dv, [0, 100, 229], seed=dk + 7 * dv)
    gpu, ref = build_both(DENSE, k, v, a, b, [0, 100, 229], True)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


@pytest.mark.parametrize("d", [32, 128])
def test_dense_build_fp32_inputs(d):
    k, v, a, b = rand_case(DENSE, 1, 2, d, d, RAGGED, seed=300 + d, bf16=False)
    gpu, ref = build_both(DENSE, k, v, a, b, RAGGED, False)
    assert_pair_close(gpu, ref, DENSE, TOL_F32)


def test_dense_build_beta_null_means_one():
    k, v, a, _ = rand_case(DENSE, 1, 2, 64, 64, [0, 130], seed=5)
    ones = np.ones(a.shape, dtype=np.float32)
    gpu, ref = build_both(DENSE, k, v, a, None, [0, 130], True)
    _, ref1 = build_both(DENSE, k, v, a, ones, [0, 130], True)
    assert np.array_equal(ref["S"], ref1["S"])
    assert_pair_close(gpu, ref1, DENSE, TOL_BF16)


@pytest.mark.parametrize("form", [SCALAR, DIAG])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("bf16", [True, False])
def test_scalar_diag_build(form, d, bf16):
    k, v, a, _ = rand_case(form, 2, 3, d, d, RAGGED, seed=400 + 10 * form + d, bf16=bf16)
    gpu, ref = build_both(form, k, v, a, None, RAGGED, bf16)
    assert_pair_close(gpu, ref, form, TOL_BF16 if bf16 else TOL_F32)


def test_one_hot_dense_build_is_bitwise():
    """k_t one-hot, beta = 1, alpha_t in {1, 1/2}, small integer v: every step of
    the chunked algorithm is exact, so the pair must equal the closed form
    S[j] = (prod of later gates) v_{t_j}, That = Diag(1[j unkeyed]) bit for bit.

    Exactness needs every intermediate to fit the split-bf16 products (about 16
    significant bits, hi + lo).  When a row is overwritten, the update mixes the
    new value with the decayed old one, so the halvings a row can accumulate
    are bounded by drawing alpha = 1/2 on about 1 token in 128."""
    from tests.test_oracle_pins import one_hot_expected
    dk = dv = 128
    H = 2
    cuts = [0, 63, 64 + 63, 64 + 63 + 500, 64 + 63 + 500 + 1024]
    N = cuts[-1]
    rng = np.random.default_rng(81)
    j = rng.integers(0, dk, size=(N, H))
    k = np.zeros((1, N, H, dk), dtype=np.float32)
    k[0, np.arange(N)[:, None], np.arange(H)[None, :], j] = 1.0
    v = rng.integers(-8, 8, size=(1, N, H, dv)).astype(np.float32)
    alpha = np.where(rng.random((1, N, H)) < 1 / 128, 0.5, 1.0).astype(np.float32)
    beta = np.ones((1, N, H), dtype=np.float32)
    gpu, ref = build_both(DENSE, k, v, alpha, beta, cuts, True)
    for s in range(len(cuts) - 1):
        S, That, lam = one_hot_expected(k.astype(np.float64), v.astype(np.float64),
                                        alpha.astype(np.float64), j, cuts[s], cuts[s + 1])
        assert np.array_equal(gpu["S0"][s, 0], S.astype(np.float32)), f"segment {s}"
        assert np.array_equal(gpu["T_hat"][s, 0], That.astype(np.float32)), f"segment {s}"
        assert lam_err(gpu["log_scale"][s, 0], lam) <= 1e-6


@pytest.mark.parametrize("d", [128, 64])
def test_one_hot_dense_build_is_bitwise_fp16(d):
    """The fp16-operand build (PIC_PREC_FP16, the kernel the dense benchmark
    times) on the exact one-hot case, bit for bit: k_t one-hot, beta = 1,
    integer v in [-8, 8), alpha = 1/2 on every 257th token (else 1).

    fp16 keeps 11 significant bits.  Every intermediate of the chunked
    algorithm is then a small integer times a power of two: the UT inverse
    has entries in {0, +-1}, the in-chunk gate ratios and chunk decays are
    powers of two, That's entries are 0 or 1 (its power-of-two column scale
    is exact), and a state row mixes values whose exponents differ by at most
    the halvings of one segment (at most 4 here), so 4 + 4 + 1 bits suffice.
    Cuts give tails of 63, 64, 65 and 1 tokens, an empty segment and a long
    one of 1024 tokens."""
    from tests.test_oracle_pins import one_hot_expected
    dk = dv = d
    H = 2
    cuts = [0, 63, 127, 127, 192, 193, 193 + 1024]
    N = cuts[-1]
    rng = np.random.default_rng(82 + d)
    j = rng.integers(0, dk, size=(N, H))
    k = np.zeros((1, N, H, dk), dtype=np.float32)
    k[0, np.arange(N)[:, None], np.arange(H)[None, :], j] = 1.0
    v = rng.integers(-8, 8, size=(1, N, H, dv)).astype(np.float32)
    t = np.arange(N)
    alpha = np.broadcast_to(np.where(t % 257 == 100, 0.5, 1.0)[None, :, None],
                            (1, N, H)).astype(np.float32)
    beta = np.ones((1, N, H), dtype=np.float32)
    gpu, _ = build_both(DENSE, k, v, alpha, beta, cuts, True, precision=1)
    for s in range(len(cuts) - 1):
        S, That, lam = one_hot_expected(k.astype(np.float64), v.astype(np.float64),
                                        alpha.astype(np.float64), j, cuts[s], cuts[s + 1])
        assert np.array_equal(gpu["S0"][s, 0], S.astype(np.float32)), f"segment {s}"
        assert np.array_equal(gpu["T_hat"][s, 0], That.astype(np.float32)), f"segment {s}"
        assert lam_err(gpu["log_scale"][s, 0], lam) <= 1e-6


def test_query_is_not_read():
    k, v, a, b = rand_case(DENSE, 1, 2, 64, 64, [0, 70], seed=9)
    q1 = np.zeros_like(k)
    q2 = np.random.default_rng(1).standard_normal(k.shape).astype(np.float32)
    g1, _ = build_both(DENSE, k, v, a, b, [0, 70], True, q=q1)
    g2, _ = build_both(DENSE, k, v, a, b, [0, 70], True, q=q2)
    for key in g1:
        assert np.array_equal(g1[key], g2[key])


def test_build_is_deterministic():
    import hybrid_caching_amd as pic
    import torch
    k, v, a, b = rand_case(DENSE, 2, 4, 128, 128, RAGGED, seed=11)
    args = (DENSE, to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16), to_dev(a), to_dev(b),
            RAGGED)
    o1 = pic.pic_segment_build(*args)
    o2 = pic.pic_segment_build(*args)
    torch.cuda.synchronize()
    for key in o1:
        assert torch.equal(o1[key], o2[key])


# --------------------------------------------------------------------------
# compose / naive add
# --------------------------------------------------------------------------

def random_pool(form, P, B, H, dk, dv, seed, lam_range=(-2.0, 0.0)):
    rng = np.random.default_rng(seed)
    lam_shape = (P, B, H, dk) if form == DIAG else (P, B, H)
    lam = rng.uniform(*lam_range, size=lam_shape).astype(np.float32)
    That = None
    if form == DENSE:
        # products of a few reflector-like factors: norm <= 1, not symmetric
        That = np.empty((P, B, H, dk, dk), dtype=np.float32)
        for idx in np.ndindex(P, B, H):
            M = np.eye(dk)
            for _ in range(3):
                x = rng.standard_normal(dk)
                x /= np.linalg.norm(x)
                M = (np.eye(dk) - rng.uniform(0, 1) * np.outer(x, x)) @ M
            That[idx] = M
    S = rng.standard_normal((P, B, H, dk, dv)).astype(np.float32)
    return lam, That, S


CHAINS = ([0, 5, 5, 12, 13], [3, 0, 7, 7, 1, 2, 3, 4, 5, 6, 8, 9, 0])


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("with_sin", [False, True])
def test_compose_matches_oracle(form, d, with_sin):
    import hybrid_caching_amd as pic
    P, B, H = 10, 2, 3
    lam, That, S = random_pool(form, P, B, H, d, d, seed=500 + d + form)
    off, idx = CHAINS
    R = len(off) - 1
    S_in = synth.random_state((R, B, H, d, d), seed=3) if with_sin else None
    out = pic.pic_compose(form, to_dev(lam), to_dev(That), to_dev(S), off, idx, to_dev(S_in))
    ref = oracle.compose(form, lam, That, S, off, idx, S_in)
    e = max_rel_units(out.cpu().numpy(), ref)
    report(f"compose err {e:.3e}")
    assert e <= TOL_F32
    nv = pic.pic_naive_add(to_dev(S), off, idx, to_dev(S_in))
    ref_nv = oracle.naive_add(S, off, idx, S_in)
    assert max_rel_units(nv.cpu().numpy(), ref_nv) <= 1e-6


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
@pytest.mark.parametrize("d", [32, 128])
def test_chain_pair_matches_oracle(form, d):
    """The chain's own pair (sum of log scales; That_pn ... That_p1 for the
    dense form), including an empty chain (0, I) and repeated entries."""
    import hybrid_caching_amd as pic
    P, B, H = 10, 2, 3
    lam, That, S = random_pool(form, P, B, H, d, d, seed=900 + d + form)
    off, idx = CHAINS
    S_out, lam_out, T_out = pic.pic_compose(form, to_dev(lam), to_dev(That), to_dev(S), off,
                                            idx, want_pair=True)
    ref_S, ref_lam, ref_T = oracle.compose(form, lam, That, S, off, idx, want_pair=True)
    assert max_rel_units(S_out.cpu().numpy(), ref_S) <= TOL_F32
    el = lam_err(lam_out.cpu().numpy(), ref_lam)
    assert el <= 1e-5, el
    assert np.all(lam_out.cpu().numpy()[1] == 0.0)  # empty chain: lambda = 0
    if form == DENSE:
        got_T = T_out.cpu().numpy()
        e = max_rel_units(got_T, ref_T)
        report(f"chain That err {e:.3e}")
        assert e <= TOL_F32
        assert np.array_equal(got_T[1], np.broadcast_to(np.eye(d, dtype=np.float32), got_T[1].shape))
    else:
        assert T_out is None


def test_chain_pair_composes_like_its_chain():
    """Folding a run of pairs into one pair and composing with it gives the
    same state as composing the run (associativity, the merge a sharded build
    would do)."""
    import hybrid_caching_amd as pic
    import torch
    P, B, H, d = 8, 1, 4, 128
    lam, That, S = random_pool(DENSE, P, B, H, d, d, seed=77, lam_range=(-0.05, 0.0))
    S_in = synth.random_state((1, B, H, d, d), seed=8)
    dl, dT, dS = to_dev(lam), to_dev(That), to_dev(S)
    seq = pic.pic_compose(DENSE, dl, dT, dS, [0, 8], list(range(8)), to_dev(S_in))
    S_a, l_a, T_a = pic.pic_compose(DENSE, dl, dT, dS, [0, 5], [0, 1, 2, 3, 4], want_pair=True)
    pool_l = torch.cat([l_a, dl[5:]])
    pool_T = torch.cat([T_a, dT[5:]])
    pool_S = torch.cat([S_a, dS[5:]])
    merged = pic.pic_compose(DENSE, pool_l, pool_T, pool_S, [0, 4], [0, 1, 2, 3], to_dev(S_in))
    ref = oracle.compose(DENSE, lam, That, S, [0, 8], list(range(8)), S_in)
    e_seq = max_rel_units(seq.cpu().numpy(), ref)
    e_merged = max_rel_units(merged.cpu().numpy(), ref)
    report(f"merged-chain err {e_merged:.3e} (sequential {e_seq:.3e})")
    assert e_seq <= TOL_F32 and e_merged <= TOL_F32


def test_compose_in_place_and_empty_chains():
    import hybrid_caching_amd as pic
    import torch
    lam, That, S = random_pool(DENSE, 4, 1, 2, 64, 64, seed=1)
    off, idx = [0, 0, 2, 2], [1, 3]
    S_in = synth.random_state((3, 1, 2, 64, 64), seed=4)
    buf = to_dev(S_in)
    pic.pic_compose(DENSE, to_dev(lam), to_dev(That), to_dev(S), off, idx, buf, out=buf)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    ref = oracle.compose(DENSE, lam, That, S, off, idx, S_in)
    assert np.array_equal(got[0], S_in[0]) and np.array_equal(got[2], S_in[2])
    assert max_rel_units(got, ref) <= TOL_F32


def test_permutation_chain_compose_is_bitwise():
    """That = permutation matrices, lambda = 0, small-integer states: every
    product is exact, so the GPU must match the oracle bit for bit."""
    import hybrid_caching_amd as pic
    rng = np.random.default_rng(91)
    P, B, H, d = 256, 2, 4, 128
    That = np.zeros((P, B, H, d, d), dtype=np.float32)
    for idx in np.ndindex(P, B, H):
        That[idx][np.arange(d), rng.permutation(d)] = 1.0
    lam = np.zeros((P, B, H), dtype=np.float32)
    S = rng.integers(-4, 5, size=(P, B, H, d, d)).astype(np.float32)
    R = 6
    off = np.arange(R + 1) * 48
    idx = rng.integers(0, P, size=off[-1]).astype(np.int32)
    S_in = rng.integers(-4, 5, size=(R, B, H, d, d)).astype(np.float32)
    out = pic.pic_compose(DENSE, to_dev(lam), to_dev(That), to_dev(S), off, idx, to_dev(S_in))
    ref = oracle.compose(DENSE, lam, That, S, off, idx, S_in)
    assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))


# --------------------------------------------------------------------------
# split + compose equals the unsplit recurrence, with slow gates (T matters)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
def test_split_compose_equals_unsplit_slow_gates(form):
    import hybrid_caching_amd as pic
    import torch
    B, H, d = 1, 4, 128
    cuts = [0, 300, 301, 700, 1024]
    k, v, a, b = rand_case(form, B, H, d, d, cuts, seed=700 + form, alpha=(0.999, 1.0),
                           beta=(0.0, 0.05))
    if form == DIAG:
        a = np.clip(a ** 0.01, 0, 1).astype(np.float32)  # slow per-channel gates
    dt = torch.bfloat16
    pair = pic.pic_segment_build(form, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), cuts)
    n = len(cuts) - 1
    out = pic.pic_compose(form, pair["log_scale"], pair.get("T_hat"), pair["S0"], [0, n],
                          list(range(n)))
    unsplit = oracle.recurrence(form, k, v, a, b)
    got = out.cpu().numpy()[0]
    # non-vacuity: the carried term is a sizeable part of the final state
    ref_pair = oracle.build(form, k, v, a, b, cuts)
    last = ref_pair["S"][-1]
    carried = (unsplit - last).reshape(H, -1)
    rho = float(np.min(np.linalg.norm(carried, axis=1)
                       / np.linalg.norm(unsplit.reshape(H, -1), axis=1)))
    assert rho >= 0.1, rho
    e = max_rel_units(got, unsplit)
    report(f"split/compose vs unsplit err {e:.3e}, rho {rho:.2f}")
    assert e <= TOL_BF16
    naive = pic.pic_naive_add(pair["S0"], [0, n], list(range(n))).cpu().numpy()[0]
    assert max_rel_units(naive, unsplit) > 10 * e  # the ablation is visibly wrong


# --------------------------------------------------------------------------
# errors: nothing is enqueued, outputs untouched
# --------------------------------------------------------------------------

def test_errors_leave_outputs_untouched():
    import hybrid_caching_amd as pic
    import torch
    k, v, a, b = rand_case(DENSE, 1, 2, 64, 64, [0, 100], seed=2)
    out = {"log_scale": torch.full((1, 1, 2), float("nan"), device="cuda:0"),
           "S0": torch.full((1, 1, 2, 64, 64), float("nan"), device="cuda:0"),
           "T_hat": torch.full((1, 1, 2, 64, 64), float("nan"), device="cuda:0")}
    dt = torch.bfloat16
    with pytest.raises(pic.PicError) as ei:
        pic.pic_segment_build(DENSE, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b),
                              [0, 101], out=out)
    assert ei.value.code == -3
    torch.cuda.synchronize()
    for t in out.values():
        assert torch.isnan(t).all()
    S_out = torch.full((1, 1, 2, 64, 64), float("nan"), device="cuda:0")
    with pytest.raises(pic.PicError) as ei:
        pic.pic_compose(DENSE, out["log_scale"], out["T_hat"], out["S0"], [0, 1], [1], out=S_out)
    assert ei.value.code == -4
    torch.cuda.synchronize()
    assert torch.isnan(S_out).all()


def test_back_to_back_calls_with_changing_tables():
    """150 builds and 150 composes with different plans are enqueued without
    synchronising (more calls than the library's pinned staging slots, so
    slots are reused while earlier copies may still be pending); every result
    matches the oracle for its own plan."""
    import torch
    import hybrid_caching_amd as pic
    form, B, H, d = SCALAR, 1, 2, 32
    plans = [[0, 64, 100], [0, 10, 100], [0, 100, 100], [0, 1, 50, 99, 100]]
    k, v, a, _ = rand_case(form, B, H, d, d, [0, 100], seed=77)
    kd, vd, ad = to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16), to_dev(a)
    lam, _, S = random_pool(form, 6, B, H, d, d, seed=78)
    lam_d, S_d = to_dev(lam), to_dev(S)
    chains = [([0, 2, 5], [0, 1, 2, 3, 4]), ([0, 1], [5]), ([0, 0, 3], [2, 2, 2]),
              ([0, 6], [5, 4, 3, 2, 1, 0]), ([0, 1, 2, 3], [1, 3, 5])]
    builds, composes = [], []
    for i in range(150):
        off = plans[i % len(plans)]
        builds.append((off, pic.pic_segment_build(form, kd, vd, ad, None, off)))
        coff, cidx = chains[i % len(chains)]
        composes.append((coff, cidx, pic.pic_compose(form, lam_d, None, S_d, coff, cidx, None)))
    torch.cuda.synchronize()
    ref_b = {tuple(p): oracle.build(form, k, v, a, None, p) for p in plans}
    for off, out in builds:
        ref = ref_b[tuple(off)]
        assert max_rel_units(out["S0"].cpu().numpy(), ref["S"]) <= TOL_BF16
        assert lam_err(out["log_scale"].cpu().numpy(), ref["lam"]) <= 1e-4
    ref_c = {i: oracle.compose(form, lam, None, S, c[0], c[1], None) for i, c in enumerate(chains)}
    for i, (coff, cidx, out) in enumerate(composes):
        assert max_rel_units(out.cpu().numpy(), ref_c[i % len(chains)]) <= TOL_F32


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
@pytest.mark.parametrize("n_seg", [32, 33, 70])
def test_plan_in_arguments_and_in_workspace(form, n_seg):
    """Plans of up to 32 segments travel in the kernel arguments, larger ones
    through the workspace: both sides of the boundary match the oracle
    (ragged lengths, empty segments included)."""
    rng = np.random.default_rng(900 + n_seg)
    lens = rng.integers(0, 90, size=n_seg)
    lens[::7] = 0
    offsets = [0] + list(np.cumsum(lens).astype(int))
    k, v, a, b = rand_case(form, 1, 2, 32, 32, offsets, seed=901 + form)
    gpu, ref = build_both(form, k, v, a, b, offsets, True)
    assert_pair_close(gpu, ref, form, TOL_BF16)
    if form == DENSE:
        gpu16, _ = build_both(form, k, v, a, b, offsets, True, precision=1)
        assert_pair_close(gpu16, ref, form, TOL_BF16)


@pytest.mark.parametrize("form", [SCALAR, DIAG, DENSE])
@pytest.mark.parametrize("n_req,steps", [(16, 4), (17, 3), (4, 40)])
def test_chain_tables_in_arguments_and_in_workspace(form, n_req, steps):
    """Chain tables of up to 16 requests and 64 entries travel in the kernel
    arguments, larger ones through the workspace."""
    import hybrid_caching_amd as pic
    P, B, H, d = 9, 1, 2, 32
    lam, That, S = random_pool(form, P, B, H, d, d, seed=910 + n_req)
    rng = np.random.default_rng(911 + steps)
    off = [0]
    idx = []
    for r in range(n_req):
        n = int(rng.integers(0, steps + 1)) if r % 3 else steps
        idx += list(rng.integers(0, P, size=n))
        off.append(len(idx))
    out = pic.pic_compose(form, to_dev(lam), to_dev(That), to_dev(S), off, idx, None)
    ref = oracle.compose(form, lam, That, S, off, idx, None)
    assert max_rel_units(out.cpu().numpy(), ref) <= TOL_F32
    nv = pic.pic_naive_add(to_dev(S), off, idx, None)
    assert max_rel_units(nv.cpu().numpy(), oracle.naive_add(S, off, idx, None)) <= 1e-6


@pytest.mark.parametrize("dk,dv", [(128, 64), (128, 32), (128, 96), (96, 32), (64, 16)])
def test_dense_compose_with_narrower_state(dk, dv):
    """dv < dk: the block has fewer state columns than operator rows, and the
    whole operator must still be staged (regression: half of a 128 x 128
    operator was left unstaged with a 64-column state)."""
    import hybrid_caching_amd as pic
    import torch
    rng = np.random.default_rng(dk * 7 + dv)
    P, B, H = 5, 2, 2
    lam = rng.uniform(-0.5, 0.0, size=(P, B, H)).astype(np.float32)
    T = (rng.standard_normal((P, B, H, dk, dk)) / np.sqrt(dk)).astype(np.float32)
    S = rng.standard_normal((P, B, H, dk, dv)).astype(np.float32)
    chain_off, chain_idx = [0, 3, 3, 8], [4, 0, 2, 1, 1, 3, 0, 2]
    S_in = rng.standard_normal((3, B, H, dk, dv)).astype(np.float32)
    for sin in (None, S_in):
        out, lam_c, T_c = pic.pic_compose(DENSE, to_dev(lam), to_dev(T), to_dev(S), chain_off,
                                          chain_idx, to_dev(sin), want_pair=True)
        torch.cuda.synchronize()
        want, want_l, want_T = oracle.compose(DENSE, lam, T, S, chain_off, chain_idx, sin,
                                              want_pair=True)
        e = max_rel_units(out.cpu().numpy(), want)
        e_t = max_rel_units(T_c.cpu().numpy(), want_T)
        report(f"dk {dk} dv {dv}: compose err {e:.3e}, chain That err {e_t:.3e}")
        assert e <= TOL_F32 and e_t <= TOL_F32
        assert lam_err(lam_c.cpu().numpy(), want_l) <= 1e-6
