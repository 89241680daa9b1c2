"""Parity of the HIP path with the fp64 oracle for the delta rule with
per-channel gates (KDA form, T_t = (I - beta_t k_t k_t^T) Diag(alpha_t)),
through the C ABI: the build of every (segment, layer, head) pair, compose of
KDA pairs (against the oracle's compose and the unsplit recurrence), the
chain's own pair, the plain operator, and the argument checks (KDA seam
windows are covered with the other forms in test_gpu_seams.py).

The token-by-token KDA build (PIC_PREC_FP32) computes in fp32 on the vector
units from the stored inputs, so bf16 inputs are held to the fp32 tolerance
as well (both sides read the same bf16-exact values).  The chunked build
(PIC_PREC_FP16: bf16 k/v, dk = dv = 128, fp16 matrix-core operands with fp32
accumulation and state) is held to the bf16-input contract bound, 2e-2
relative Frobenius error per unit: ragged chunk tails and empty segments,
long and many segments, slow gates, beta = NULL, shared gates against the
dense oracle, repeated calls, the overflow report outside its gate range and
the rejected shapes.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import DENSE, KDA
from tests.gpu_helpers import (TOL_BF16, TOL_F32, assert_pair_close, build_both, lam_err,
                               max_rel_units, report, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def kda_case(B, H, dk, dv, offsets, seed, bf16=True, gate=(3.0, 1.0), beta=(0.0, 1.0)):
    """Seeded KDA inputs: unit-norm keys, v ~ N(0, 1), per-channel gates
    sigmoid(N(mu, sigma)), beta ~ U(lo, hi); k, v rounded to the storage type."""
    rng = np.random.default_rng(seed)
    N = int(offsets[-1])
    k = rng.standard_normal((B, N, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, H, dv)).astype(np.float32)
    if bf16:
        k, v = synth.bf16_round(k), synth.bf16_round(v)
    z = rng.normal(gate[0], gate[1], size=(B, N, H, dk))
    a = np.clip(1.0 / (1.0 + np.exp(-z)), 1e-30, 1.0).astype(np.float32)
    b = rng.uniform(*beta, size=(B, N, H)).astype(np.float32) if beta is not None else None
    return k, v, a, b


RAGGED = [0, 15, 16, 16, 47, 48, 113]  # rounds of 16 tokens: tails of 15 / 1 / 15, an empty segment


@pytest.mark.parametrize("d", [16, 32, 64, 96, 128])
def test_kda_build_head_sizes(d):
    k, v, a, b = kda_case(2, 3, d, d, RAGGED, seed=800 + d)
    gpu, ref = build_both(KDA, k, v, a, b, RAGGED, True)
    assert_pair_close(gpu, ref, KDA, TOL_F32)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (32, 96), (16, 128)])
def test_kda_build_unequal_dims(dk, dv):
    offs = [0, 100, 229]
    k, v, a, b = kda_case(1, 2, dk, dv, offs, seed=dk + 7 * dv)
    gpu, ref = build_both(KDA, k, v, a, b, offs, True)
    assert_pair_close(gpu, ref, KDA, TOL_F32)


@pytest.mark.parametrize("d", [32, 128])
def test_kda_build_fp32_inputs(d):
    k, v, a, b = kda_case(1, 2, d, d, RAGGED, seed=900 + d, bf16=False)
    gpu, ref = build_both(KDA, k, v, a, b, RAGGED, False)
    assert_pair_close(gpu, ref, KDA, TOL_F32)


def test_kda_build_beta_null_means_one():
    k, v, a, _ = kda_case(1, 2, 64, 64, [0, 130], seed=5, beta=None)
    ones = np.ones(a.shape[:3], dtype=np.float32)
    gpu, ref = build_both(KDA, k, v, a, None, [0, 130], True)
    _, ref1 = build_both(KDA, k, v, a, ones, [0, 130], True)
    assert np.array_equal(ref["S"], ref1["S"])
    assert_pair_close(gpu, ref1, KDA, TOL_F32)


def test_kda_build_small_gates():
    """Small gates (a shared factor in (0.05, 0.2) times a per-channel one in
    (0.9, 1]) over 200 tokens: lambda falls to about -400, where T_C itself
    underflows fp32, while That stays representable, bounded (||That||_2 <= 1)
    and matched."""
    offs = [0, 200]
    rng = np.random.default_rng(31)
    k, v, _, b = kda_case(1, 2, 128, 128, offs, seed=31)
    base = rng.uniform(0.05, 0.2, size=k.shape[:3] + (1,))
    a = (base * rng.uniform(0.9, 1.0, size=k.shape)).astype(np.float32)
    gpu, ref = build_both(KDA, k, v, a, b, offs, True)
    assert_pair_close(gpu, ref, KDA, TOL_F32)
    assert np.max(gpu["log_scale"]) < -200.0
    for h in range(2):
        nrm = np.linalg.norm(gpu["T_hat"][0, 0, h].astype(np.float64), 2)
        assert 1e-20 < nrm <= 1.0 + 1e-4


def test_kda_shared_gates_match_the_dense_oracle():
    """All channels share one gate: the KDA build is the dense GDN pair."""
    offs = [0, 77, 200]
    k, v, a, b = kda_case(1, 2, 64, 64, offs, seed=44)
    a1 = a[..., 0]
    a_all = np.ascontiguousarray(np.repeat(a1[..., None], 64, axis=-1))
    gpu, _ = build_both(KDA, k, v, a_all, b, offs, True)
    ref = oracle.build(DENSE, k, v, a1, b, offs)
    assert_pair_close(gpu, ref, DENSE, TOL_F32)


def test_kda_many_segments_use_the_workspace_plan():
    """More segments than travel in the kernel arguments (40 > 32)."""
    lens = np.random.default_rng(3).integers(0, 40, size=40)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    k, v, a, b = kda_case(1, 2, 32, 32, offs, seed=45)
    gpu, ref = build_both(KDA, k, v, a, b, offs, True)
    assert_pair_close(gpu, ref, KDA, TOL_F32)


def test_kda_all_segments_empty():
    import hybrid_caching_amd as pic
    import torch
    dt = torch.bfloat16
    dev = torch.device("cuda:0")
    k = torch.zeros((1, 0, 2, 32), dtype=dt, device=dev)
    v = torch.zeros((1, 0, 2, 32), dtype=dt, device=dev)
    a = torch.zeros((1, 0, 2, 32), dtype=torch.float32, device=dev)
    out = pic.pic_segment_build(KDA, k, v, a, None, [0, 0, 0])
    torch.cuda.synchronize()
    assert torch.count_nonzero(out["log_scale"]).item() == 0
    assert torch.count_nonzero(out["S0"]).item() == 0
    eye = torch.eye(32, device=dev).expand(2, 1, 2, 32, 32)
    assert torch.equal(out["T_hat"], eye)


# --------------------------------------------------------------------------
# chunked build on the matrix cores (PIC_PREC_FP16)
# --------------------------------------------------------------------------

FP16 = 1
NONFINITE, UNSUPPORTED = -9, -6
# lengths 31, 1, 0, 65, 63, 1: a partial chunk, single tokens, an empty
# segment, two whole chunks and a 1-token tail, a whole chunk and a 31-token tail
RAGGED32 = [0, 31, 32, 32, 97, 160, 161]


def test_kda_fp16_ragged_segments():
    k, v, a, b = kda_case(2, 3, 128, 128, RAGGED32, seed=1100)
    gpu, ref = build_both(KDA, k, v, a, b, RAGGED32, True, precision=FP16)
    assert_pair_close(gpu, ref, KDA, TOL_BF16)
    # the empty segment: zero state, identity That, lambda 0
    assert not gpu["S0"][2].any() and not gpu["log_scale"][2].any()
    assert np.array_equal(gpu["T_hat"][2], np.broadcast_to(np.eye(128, dtype=np.float32),
                                                           gpu["T_hat"][2].shape))


@pytest.mark.parametrize("n", [1024, 4096])
def test_kda_fp16_long_segments(n):
    """Whole segments of the workload's length: That decays far below fp16's
    range and is carried at a power-of-two scale."""
    offs = [0, n]
    k, v, a, b = kda_case(1, 2, 128, 128, offs, seed=1200 + n)
    gpu, ref = build_both(KDA, k, v, a, b, offs, True, precision=FP16)
    assert_pair_close(gpu, ref, KDA, TOL_BF16)


def test_kda_fp16_slow_gates():
    offs = [0, 1000, 2048]
    k, v, a, b = kda_case(1, 2, 128, 128, offs, seed=1300, gate=(9.0, 1.0), beta=(0.0, 0.02))
    gpu, ref = build_both(KDA, k, v, a, b, offs, True, precision=FP16)
    assert_pair_close(gpu, ref, KDA, TOL_BF16)


def test_kda_fp16_beta_null_means_one():
    offs = [0, 70, 130]
    k, v, a, _ = kda_case(1, 2, 128, 128, offs, seed=1400, beta=None)
    ones = np.ones(a.shape[:3], dtype=np.float32)
    gpu, _ = build_both(KDA, k, v, a, None, offs, True, precision=FP16)
    ref1 = oracle.build(KDA, k, v, a, ones, offs)
    assert_pair_close(gpu, ref1, KDA, TOL_BF16)


def test_kda_fp16_shared_gates_match_the_dense_oracle():
    offs = [0, 77, 200]
    k, v, a, b = kda_case(1, 2, 128, 128, offs, seed=1500)
    a1 = a[..., 0]
    a_all = np.ascontiguousarray(np.repeat(a1[..., None], 128, axis=-1))
    gpu, _ = build_both(KDA, k, v, a_all, b, offs, True, precision=FP16)
    ref = oracle.build(DENSE, k, v, a1, b, offs)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


def test_kda_fp16_many_segments_use_the_workspace_plan():
    lens = np.random.default_rng(1600).integers(0, 80, size=40)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    k, v, a, b = kda_case(1, 2, 128, 128, offs, seed=1601)
    gpu, ref = build_both(KDA, k, v, a, b, offs, True, precision=FP16)
    assert_pair_close(gpu, ref, KDA, TOL_BF16)


def test_kda_fp16_repeated_calls_are_bit_identical_and_flag_clear():
    import hybrid_caching_amd as pic
    import torch
    offs = [0, 50, 129]
    k, v, a, b = kda_case(1, 2, 128, 128, offs, seed=1700)
    dt = torch.bfloat16
    args = (to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), offs)
    try:
        pic.pic_nonfinite_check()
    except pic.PicError:
        pass
    x = pic.pic_segment_build(KDA, *args, precision=FP16, check_finite=True)
    y = pic.pic_segment_build(KDA, *args, precision=FP16, check_finite=True)
    torch.cuda.synchronize()
    for key in x:
        assert torch.equal(x[key], y[key]), key


def test_kda_fp16_fast_gates_leave_the_range_and_are_reported():
    """Gates near 0.1 in every channel: a 16-token gate product is about
    1e-16, far outside fp16's range, so the chunked build overflows and its
    report says so; the fp32 build of the same inputs matches the oracle."""
    import hybrid_caching_amd as pic
    import torch
    offs = [0, 64]
    rng = np.random.default_rng(1800)
    k, v, _, b = kda_case(1, 1, 128, 128, offs, seed=1801)
    a = rng.uniform(0.05, 0.2, size=k.shape).astype(np.float32)
    try:
        pic.pic_nonfinite_check()
    except pic.PicError:
        pass
    dt = torch.bfloat16
    with pytest.raises(pic.PicError) as err:
        pic.pic_segment_build(KDA, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), offs,
                              precision=FP16, check_finite=True)
    assert err.value.code == NONFINITE
    pic.pic_nonfinite_check()  # cleared by the report
    gpu, ref = build_both(KDA, k, v, a, b, offs, True)
    assert_pair_close(gpu, ref, KDA, TOL_F32)


@pytest.mark.parametrize("dk,dv,bf16", [(64, 64, True), (128, 64, True), (128, 128, False)])
def test_kda_fp16_rejects_other_shapes(dk, dv, bf16):
    import hybrid_caching_amd as pic
    import torch
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = torch.device("cuda:0")
    k = torch.zeros((1, 8, 1, dk), dtype=dt, device=dev)
    v = torch.zeros((1, 8, 1, dv), dtype=dt, device=dev)
    a = torch.ones((1, 8, 1, dk), dtype=torch.float32, device=dev)
    with pytest.raises(pic.PicError) as err:
        pic.pic_segment_build(KDA, k, v, a, None, [0, 8], precision=FP16)
    assert err.value.code == UNSUPPORTED


# --------------------------------------------------------------------------
# compose of KDA pairs
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [32, 128])
def test_kda_compose_equals_unsplit_recurrence(d):
    """Pairs built on the GPU, composed on the GPU, against the recurrence
    over the concatenated tokens (the identity the split must keep), from a
    zero and from a random incoming state; and the chain's own pair against
    the pair of the whole token range."""
    import hybrid_caching_amd as pic
    import torch
    offs = [0, 50, 50, 131, 200]
    k, v, a, b = kda_case(2, 2, d, d, offs, seed=60 + d, gate=(6.0, 1.0))
    dt = torch.bfloat16
    pair = pic.pic_segment_build(KDA, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), offs)
    n = len(offs) - 1
    S_in = synth.random_state((1, 2, 2, d, d), seed=61)
    for sin in (None, S_in):
        out, lam_c, T_c = pic.pic_compose(KDA, pair["log_scale"], pair["T_hat"], pair["S0"],
                                          [0, n], list(range(n)), to_dev(sin), want_pair=True)
        torch.cuda.synchronize()
        unsplit = oracle.recurrence(KDA, k, v, a, b, None if sin is None else sin[0])
        e = max_rel_units(out.cpu().numpy()[0], unsplit)
        report(f"d {d} compose vs unsplit: {e:.3e}")
        assert e <= TOL_F32
    whole = oracle.build(KDA, k, v, a, b, [0, offs[-1]])
    e_t = max_rel_units(T_c.cpu().numpy(), whole["That"])
    e_l = lam_err(lam_c.cpu().numpy(), whole["lam"])
    report(f"d {d} chain pair: That err {e_t:.3e}, lambda err {e_l:.3e}")
    assert e_t <= TOL_F32 and e_l <= 1e-5


def test_kda_compose_against_oracle_compose():
    """Chains in any order over a pool of KDA pairs (oracle-built pairs as
    the pool, so only compose is under test), with repeats and an empty chain."""
    import hybrid_caching_amd as pic
    import torch
    offs = [0, 40, 90, 90, 160]
    k, v, a, b = kda_case(2, 3, 64, 96, offs, seed=70, gate=(8.0, 1.0))
    ref = oracle.build(KDA, k, v, a, b, offs)
    f32 = lambda x: to_dev(np.asarray(x, dtype=np.float32))
    chain_off, chain_idx = [0, 3, 3, 7], [2, 0, 3, 1, 1, 3, 0]
    S_in = synth.random_state((3, 2, 3, 64, 96), seed=71)
    out = pic.pic_compose(KDA, f32(ref["lam"]), f32(ref["That"]), f32(ref["S"]), chain_off,
                          chain_idx, to_dev(S_in))
    torch.cuda.synchronize()
    want = oracle.compose(KDA, ref["lam"], ref["That"], ref["S"], chain_off, chain_idx, S_in)
    e = max_rel_units(out.cpu().numpy(), want)
    report(f"compose vs oracle compose: {e:.3e}")
    assert e <= TOL_F32


def test_kda_materialize_T():
    import hybrid_caching_amd as pic
    import torch
    offs = [0, 30, 64]
    k, v, a, b = kda_case(1, 2, 32, 32, offs, seed=80)
    dt = torch.bfloat16
    pair = pic.pic_segment_build(KDA, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), offs)
    T = pic.pic_materialize_T(KDA, pair["log_scale"], pair["T_hat"])
    torch.cuda.synchronize()
    ref_T = oracle.build(KDA, k, v, a, b, offs, want_T=True)["T"]
    assert max_rel_units(T.cpu().numpy(), ref_T) <= TOL_F32


def test_kda_build_without_T_hat_is_rejected_before_any_work():
    """A KDA build needs That; the call fails on the host before anything is
    enqueued and leaves the outputs untouched."""
    import hybrid_caching_amd as pic
    import torch
    dev = torch.device("cuda:0")
    k = torch.zeros((1, 8, 1, 16), dtype=torch.bfloat16, device=dev)
    a = torch.ones((1, 8, 1, 16), dtype=torch.float32, device=dev)
    out = {"log_scale": torch.full((1, 1, 1), 7.0, device=dev),
           "S0": torch.full((1, 1, 1, 16, 16), 7.0, device=dev)}
    with pytest.raises(pic.PicError):
        pic.pic_segment_build(KDA, k, k, a, None, [0, 8], out=out)
    torch.cuda.synchronize()
    assert bool((out["S0"] == 7.0).all()) and bool((out["log_scale"] == 7.0).all())
