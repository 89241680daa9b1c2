"""Parity of the dense build at fp16 operand precision (PIC_PREC_FP16: one
fp16 matrix-core product per operand pair, fp32 accumulation and state) with
the fp64 oracle, through the C ABI, on seeded bf16 inputs: every supported
head size with ragged chunk tails and empty segments, unequal key / value
sizes, long segments (4096 and 8192 tokens, where the ungated product That
decays far below fp16's range and must be carried at a power-of-two scale),
slow gates, beta = NULL, and the bookkeeping properties (queries never read,
repeated calls bit-identical).  The contract bound with bf16 inputs is a
relative Frobenius error of 2e-2 per unit; the errors are reported.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import DENSE
from tests.gpu_helpers import TOL_BF16, assert_pair_close, build_both, report, to_dev

pytestmark = pytest.mark.gpu
FP16 = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()  # fails loudly if the HIP library is missing


def dense_case(B, H, dk, dv, offsets, seed, alpha=(0.9, 1.0), beta=(0.0, 1.0)):
    """Seeded dense inputs: k rows L2-normalised in fp32, then k, v rounded to bf16."""
    rng = np.random.default_rng(seed)
    N = int(offsets[-1])
    k = rng.standard_normal((B, N, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, H, dv)).astype(np.float32)
    k, v = synth.bf16_round(k), synth.bf16_round(v)
    a = rng.uniform(*alpha, size=(B, N, H)).astype(np.float32)
    b = rng.uniform(*beta, size=(B, N, H)).astype(np.float32)
    return k, v, a, b


RAGGED = [0, 63, 127, 127, 300, 364, 500]  # tails of 63 / 64 / 45 / 1 tokens, an empty segment


@pytest.mark.parametrize("d", [16, 32, 48, 64, 96, 128])
def test_fp16_head_sizes(d):
    k, v, a, b = dense_case(2, 3, d, d, RAGGED, seed=700 + d)
    gpu, ref = build_both(DENSE, k, v, a, b, RAGGED, True, precision=FP16)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (32, 96), (112, 16)])
def test_fp16_unequal_dims(dk, dv):
    offs = [0, 100, 229, 229, 420]
    k, v, a, b = dense_case(1, 2, dk, dv, offs, seed=11 * dk + dv)
    gpu, ref = build_both(DENSE, k, v, a, b, offs, True, precision=FP16)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


@pytest.mark.parametrize("L", [4096, 8192])
def test_fp16_long_segments(L):
    """That decays to ~1e-4 (4096) and ~5e-9 (8192) in norm along the segment."""
    offs = [0, L, L + 1000]
    k, v, a, b = dense_case(1, 2, 128, 128, offs, seed=L)
    gpu, ref = build_both(DENSE, k, v, a, b, offs, True, precision=FP16)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


def test_fp16_slow_gates():
    """alpha near 1 and small beta: S accumulates over the whole segment."""
    offs = [0, 2048, 4096]
    k, v, a, b = dense_case(1, 2, 128, 128, offs, seed=31, alpha=(0.9995, 1.0), beta=(0.0, 0.02))
    gpu, ref = build_both(DENSE, k, v, a, b, offs, True, precision=FP16)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


def test_fp16_beta_null_means_one():
    offs = [0, 130, 300]
    k, v, a, _ = dense_case(1, 2, 64, 64, offs, seed=5)
    ones = np.ones(a.shape, dtype=np.float32)
    gpu, _ = build_both(DENSE, k, v, a, None, offs, True, precision=FP16)
    _, ref1 = build_both(DENSE, k, v, a, ones, offs, True)
    assert_pair_close(gpu, ref1, DENSE, TOL_BF16)


def test_fp16_many_short_segments():
    rng = np.random.default_rng(9)
    lens = rng.integers(0, 150, size=120)
    offs = np.concatenate([[0], np.cumsum(lens)])
    k, v, a, b = dense_case(1, 2, 128, 128, offs, seed=77)
    gpu, ref = build_both(DENSE, k, v, a, b, offs, True, precision=FP16)
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


def test_fp16_queries_unread_and_deterministic():
    """Changing q leaves every output bit-identical; so does calling again."""
    import hybrid_caching_amd as pic
    import torch
    offs = [0, 200, 333]
    k, v, a, b = dense_case(2, 2, 128, 128, offs, seed=3)
    dt = torch.bfloat16
    args = (DENSE, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), offs)
    q1 = to_dev(np.zeros_like(k), dt)
    q2 = to_dev(np.random.default_rng(1).standard_normal(k.shape).astype(np.float32), dt)
    o1 = pic.pic_segment_build(*args, q=q1, precision=FP16)
    o2 = pic.pic_segment_build(*args, q=q2, precision=FP16)
    o3 = pic.pic_segment_build(*args, precision=FP16)
    torch.cuda.synchronize()
    for key in o1:
        assert torch.equal(o1[key], o2[key]) and torch.equal(o1[key], o3[key]), key


def test_fp16_all_segments_empty():
    import hybrid_caching_amd as pic
    import torch
    dev = torch.device("cuda:0")
    k = torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16, device=dev)
    v = torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16, device=dev)
    a = torch.zeros((2, 0, 3), dtype=torch.float32, device=dev)
    pair = pic.pic_segment_build(DENSE, k, v, a, None, [0, 0, 0], precision=FP16)
    torch.cuda.synchronize()
    assert torch.all(pair["S0"] == 0) and torch.all(pair["log_scale"] == 0)
    eye = torch.eye(64, device=dev).expand_as(pair["T_hat"])
    assert torch.equal(pair["T_hat"], eye)


def test_fp16_rejects_other_combinations():
    import hybrid_caching_amd as pic
    import torch
    from hybrid_caching_amd._lib import PicError
    offs = [0, 64]
    k, v, a, b = dense_case(1, 1, 32, 32, offs, seed=1)
    with pytest.raises(PicError):  # fp32 inputs
        pic.pic_segment_build(DENSE, to_dev(k), to_dev(v), to_dev(a), to_dev(b), offs,
                              precision=FP16)
    with pytest.raises(PicError):  # scalar form
        pic.pic_segment_build(oracle.SCALAR, to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16),
                              to_dev(a), None, offs, precision=FP16)
    report("fp16 precision rejects fp32 inputs and non-dense forms")
