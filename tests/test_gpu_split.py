"""The split build (pic_segment_build_split) through the C ABI: every segment
cut into pieces of whole 64-token chunks, the pieces' pairs built and merged
in token order by the chain-pair compose, so a launch with few (segment,
layer, head) units fills the GPU.  Checked bit for bit on the exact one-hot
case (the pieces' boundaries and the merge order), against the fp64 oracle
for every form and precision with ragged, empty and short segments, with slow
gates (where the merge's T products carry a sizeable part of the state), and
against the plain build on the same inputs.
"""
import numpy as np
import pytest

import oracle
from oracle import DENSE, DIAG, KDA, SCALAR
from tests.gpu_helpers import (TOL_BF16, TOL_F32, assert_pair_close, lam_err, max_rel_units,
                               report, to_dev)
from tests.test_gpu_kda import kda_case
from tests.test_gpu_parity import rand_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def split_both(form, k, v, a, b, offs, bf16, split, precision=0):
    import hybrid_caching_amd as pic
    import torch
    dt = torch.bfloat16 if bf16 else torch.float32
    out = pic.pic_segment_build(form, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), offs,
                                precision=precision, split=split)
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in out.items()}
    return gpu, oracle.build(form, k, v, a, b, offs)


# lengths 0, 1, 63, 65, 200, 1000, 3000: empty, shorter than one chunk, one
# chunk, two chunks, four, sixteen and 47 chunks (more than the pieces)
RAGGED = [0, 0, 1, 64, 129, 329, 1329, 4329]


@pytest.mark.parametrize("precision", [0, 1])
def test_split_one_hot_is_bitwise(precision):
    """k_t one-hot, beta = 1, alpha = 1, integer v: every piece and every
    merge step is exact, so the pairs must equal the closed form bit for bit
    (a later piece overwrites the rows it keys, That = Diag(1[j unkeyed]),
    lambda = 0); a wrong piece boundary or merge order changes rows."""
    from tests.test_oracle_pins import one_hot_expected
    d = 128
    H = 2
    cuts = [0, 63, 127, 127, 127 + 1000, 127 + 1000 + 2048]
    N = cuts[-1]
    rng = np.random.default_rng(1900 + precision)
    j = rng.integers(0, d, size=(N, H))
    k = np.zeros((1, N, H, d), dtype=np.float32)
    k[0, np.arange(N)[:, None], np.arange(H)[None, :], j] = 1.0
    v = rng.integers(-8, 8, size=(1, N, H, d)).astype(np.float32)
    alpha = np.ones((1, N, H), dtype=np.float32)
    beta = np.ones((1, N, H), dtype=np.float32)
    gpu, _ = split_both(DENSE, k, v, alpha, beta, cuts, True, split=5, precision=precision)
    for s in range(len(cuts) - 1):
        S, That, lam = one_hot_expected(k.astype(np.float64), v.astype(np.float64),
                                        alpha.astype(np.float64), j, cuts[s], cuts[s + 1])
        assert np.array_equal(gpu["S0"][s, 0], S.astype(np.float32)), f"segment {s}"
        assert np.array_equal(gpu["T_hat"][s, 0], That.astype(np.float32)), f"segment {s}"
        assert np.all(gpu["log_scale"][s] == 0.0)


@pytest.mark.parametrize("form,bf16,precision,tol", [
    (SCALAR, True, 0, TOL_F32), (DIAG, True, 0, TOL_F32), (DENSE, False, 0, TOL_F32),
    (DENSE, True, 0, TOL_F32), (DENSE, True, 1, TOL_BF16), (KDA, True, 0, TOL_F32),
    (KDA, True, 1, TOL_BF16)])
@pytest.mark.parametrize("split", [2, 5])
def test_split_matches_oracle(form, bf16, precision, tol, split):
    if form == KDA:
        k, v, a, b = kda_case(1, 2, 128, 128, RAGGED, seed=2000 + split, bf16=bf16)
    else:
        k, v, a, b = rand_case(form, 1, 2, 128, 128, RAGGED, seed=2000 + 10 * form + split,
                               bf16=bf16)
    gpu, ref = split_both(form, k, v, a, b, RAGGED, bf16, split, precision)
    report(f"form {form} bf16 {bf16} precision {precision} split {split}:")
    assert_pair_close(gpu, ref, form, tol)


@pytest.mark.parametrize("form", [DENSE, KDA])
def test_split_slow_gates_exercises_the_merge(form):
    """Slow gates and small erase strengths over 6144 tokens: the earlier
    pieces' states reach the end through the later pieces' T (rho >= 0.1 for
    the piece boundary in the middle), so the merge's products matter."""
    offs = [0, 6144]
    if form == KDA:
        k, v, a, b = kda_case(1, 2, 128, 128, offs, seed=2100, gate=(9.0, 1.0), beta=(0.0, 0.02))
    else:
        k, v, a, b = rand_case(DENSE, 1, 2, 128, 128, offs, seed=2101, alpha=(0.9995, 1.0),
                               beta=(0.0, 0.02))
    for precision, tol in ((0, TOL_F32), (1, TOL_BF16)):
        gpu, ref = split_both(form, k, v, a, b, offs, True, 6, precision)
        report(f"form {form} precision {precision} slow gates, 6 pieces:")
        assert_pair_close(gpu, ref, form, tol)
    half = oracle.build(form, k, v, a, b, [0, 3072, 6144])
    # rho of the middle boundary: |T(C2) S(C1)| / |S(C1.C2)|
    T2 = np.exp(half["lam"][1])[..., None, None] * half["That"][1]
    TS = np.einsum("bhij,bhjk->bhik", T2, half["S"][0])
    rho = np.linalg.norm(TS) / np.linalg.norm(TS + half["S"][1])
    report(f"form {form}: rho at the middle boundary {rho:.3f}")
    assert rho >= 0.1


def test_split_equals_plain_build():
    """The same inputs built whole and in pieces (fp16 operands): equal up to
    the rounding of the merge."""
    import hybrid_caching_amd as pic
    import torch
    offs = [0, 4096, 4096 + 2500]
    k, v, a, b = rand_case(DENSE, 2, 3, 128, 128, offs, seed=2200)
    dt = torch.bfloat16
    args = (to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), offs)
    whole = pic.pic_segment_build(DENSE, *args, precision=1)
    parts = pic.pic_segment_build(DENSE, *args, precision=1, split=4)
    torch.cuda.synchronize()
    e_s = max_rel_units(parts["S0"].cpu().numpy(), whole["S0"].cpu().numpy())
    e_t = max_rel_units(parts["T_hat"].cpu().numpy(), whole["T_hat"].cpu().numpy())
    e_l = lam_err(parts["log_scale"].cpu().numpy(), whole["log_scale"].cpu().numpy())
    report(f"split vs whole: S {e_s:.2e}, That {e_t:.2e}, lambda {e_l:.2e}")
    assert e_s <= TOL_BF16 and e_t <= TOL_BF16 and e_l <= 1e-5


def test_split_few_units_long_segment():
    """The case the split is for: one 16384-token segment, one layer, four
    heads (4 units), fp16 operands, cut into 16 pieces."""
    import hybrid_caching_amd as pic
    offs = [0, 16384]
    assert pic.suggest_split(1, 4, offs) == 16
    k, v, a, b = rand_case(DENSE, 1, 4, 128, 128, offs, seed=2300)
    gpu, ref = split_both(DENSE, k, v, a, b, offs, True, 16, precision=1)
    report("one segment of 16384 tokens, 4 heads, 16 pieces:")
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)
