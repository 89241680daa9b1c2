"""Parity of the HIP prefill with per-token outputs (pic_segment_prefill:
dense form, bf16 q/k/v, fp16 operand precision) with the fp64 oracle, through
the C ABI: every token's output o_t = S_t^T q_t of the independent prefill of
each segment and the segment's pair, with and without That; head sizes 16-128,
unequal dk / dv, ragged tails and empty segments; bit for bit on an exact
one-hot case; the pair equal to the build's; sampled units at the full
segment length of the 30-layer workload.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import DENSE
from tests.gpu_helpers import (TOL_BF16, assert_pair_close, lam_err, max_rel_units, report,
                               to_dev)
from tests.test_gpu_parity import RAGGED, rand_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def _prefill_both(q, k, v, a, b, offsets, track_T=True):
    import hybrid_caching_amd as pic
    import torch
    bf = torch.bfloat16
    out = pic.pic_segment_prefill(to_dev(q, bf), to_dev(k, bf), to_dev(v, bf), to_dev(a),
                                  to_dev(b), offsets, track_T=track_T)
    torch.cuda.synchronize()
    gpu = {key: val.float().cpu().numpy() for key, val in out.items()}
    ref = oracle.prefill(DENSE, q, k, v, a, b, offsets)
    return gpu, ref


def _o_err(got, ref):
    # relative Frobenius error per (layer, head) over all its tokens
    return max_rel_units(np.transpose(got, (0, 2, 1, 3)), np.transpose(ref, (0, 2, 1, 3)))


def _q(shape, seed):
    return synth.bf16_round(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("track_T", [True, False])
@pytest.mark.parametrize("d", [16, 32, 64, 96, 128])
def test_prefill_matches_oracle(d, track_T):
    k, v, a, b = rand_case(DENSE, 2, 3, d, d, RAGGED, seed=700 + d)
    q = _q(k.shape, 701 + d)
    gpu, ref = _prefill_both(q, k, v, a, b, RAGGED, track_T)
    e = _o_err(gpu["O"], ref["O"])
    report(f"prefill d {d} track_T {track_T}: output err {e:.3e}")
    assert e <= TOL_BF16
    if track_T:
        assert_pair_close(gpu, ref, DENSE, TOL_BF16)
    else:
        assert "T_hat" not in gpu
        assert max_rel_units(gpu["S0"], ref["S"]) <= TOL_BF16
        assert lam_err(gpu["log_scale"], ref["lam"]) <= 1e-4


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (32, 96)])
def test_prefill_unequal_dims(dk, dv):
    cuts = [0, 100, 229]
    k, v, a, b = rand_case(DENSE, 1, 2, dk, dv, cuts, seed=dk + 3 * dv)
    q = _q(k.shape, dk * dv)
    gpu, ref = _prefill_both(q, k, v, a, b, cuts)
    e = _o_err(gpu["O"], ref["O"])
    report(f"prefill dk {dk} dv {dv}: output err {e:.3e}")
    assert e <= TOL_BF16
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


def test_prefill_slow_gates_long_segments():
    """Slowly decaying gates over two long segments: the state carries far,
    and the lazy decay passes through many lazy and eager steps."""
    cuts = [0, 1500, 3000]
    k, v, a, b = rand_case(DENSE, 1, 2, 128, 128, cuts, seed=77, alpha=(0.999, 1.0),
                           beta=(0.0, 0.05))
    q = _q(k.shape, 78)
    gpu, ref = _prefill_both(q, k, v, a, b, cuts)
    e = _o_err(gpu["O"], ref["O"])
    report(f"prefill slow gates: output err {e:.3e}")
    assert e <= TOL_BF16
    assert_pair_close(gpu, ref, DENSE, TOL_BF16)


def test_prefill_pair_matches_build_and_that_is_optional():
    """The prefill's pair agrees with the build's (two kernels, both near the
    oracle); leaving That out changes neither the outputs nor S(C|0) (bit for
    bit: the S chain does not read That); beta = None means beta = 1."""
    import hybrid_caching_amd as pic
    import torch
    cuts = [0, 65, 65, 190]
    k, v, a, _ = rand_case(DENSE, 2, 2, 64, 64, cuts, seed=91)
    q = _q(k.shape, 92)
    bf = torch.bfloat16
    ones = np.ones(a.shape, dtype=np.float32)
    dq, dk_, dv_, da = to_dev(q, bf), to_dev(k, bf), to_dev(v, bf), to_dev(a)
    pf = pic.pic_segment_prefill(dq, dk_, dv_, da, None, cuts)
    pf1 = pic.pic_segment_prefill(dq, dk_, dv_, da, to_dev(ones), cuts)
    pf0 = pic.pic_segment_prefill(dq, dk_, dv_, da, None, cuts, track_T=False)
    bd = pic.pic_segment_build(DENSE, dk_, dv_, da, None, cuts, precision=1)
    torch.cuda.synchronize()
    for key in ("log_scale", "T_hat", "S0", "O"):
        assert torch.equal(pf[key], pf1[key]), key
    for key in ("log_scale", "S0", "O"):
        assert torch.equal(pf[key], pf0[key]), key
    assert "T_hat" not in pf0
    gp = {key: t.cpu().numpy() for key, t in pf.items() if key != "O"}
    ref = {"lam": bd["log_scale"].cpu().numpy().astype(np.float64),
           "That": bd["T_hat"].cpu().numpy().astype(np.float64),
           "S": bd["S0"].cpu().numpy().astype(np.float64)}
    assert_pair_close(gp, ref, DENSE, 5e-3)


def test_prefill_one_hot_is_bitwise():
    """k_t and q_t one-hot, beta = 1, alpha = 1/2 on every 257th token (else
    1; at most 3 halvings per segment), integer v in [-8, 8): every state entry is a small integer times a
    power of two, so the outputs (rows of the state, exact in bf16) and the
    pair must equal the fp64 oracle bit for bit.  Cuts give tails of 63, 64,
    65 and 1 tokens and an empty segment."""
    import hybrid_caching_amd as pic
    import torch
    dk = dv = 128
    H = 2
    cuts = [0, 63, 127, 127, 192, 193, 193 + 700]
    N = cuts[-1]
    rng = np.random.default_rng(93)
    jk = rng.integers(0, dk, size=(N, H))
    jq = rng.integers(0, dk, size=(N, H))
    k = np.zeros((1, N, H, dk), dtype=np.float32)
    q = np.zeros((1, N, H, dk), dtype=np.float32)
    k[0, np.arange(N)[:, None], np.arange(H)[None, :], jk] = 1.0
    q[0, np.arange(N)[:, None], np.arange(H)[None, :], jq] = 1.0
    v = rng.integers(-8, 8, size=(1, N, H, dv)).astype(np.float32)
    t = np.arange(N)
    a = np.broadcast_to(np.where(t % 257 == 40, 0.5, 1.0)[None, :, None], (1, N, H)).astype(np.float32)
    b = np.ones((1, N, H), dtype=np.float32)
    gpu, ref = _prefill_both(q, k, v, a, b, cuts)
    want = synth.bf16_round(ref["O"].astype(np.float32))
    assert np.array_equal(gpu["O"], want)
    assert np.array_equal(gpu["S0"], ref["S"].astype(np.float32))
    assert np.array_equal(gpu["T_hat"], ref["That"].astype(np.float32))


@pytest.mark.timeout(400)
def test_prefill_full_length_sampled():
    """Two layers of the 30-layer workload at its full segment length (32
    segments of 4096 tokens, 32 heads, d = 128); sampled (layer, head,
    segment) units against the oracle run on those units' tokens alone."""
    import hybrid_caching_amd as pic
    import torch
    w = synth.scaled(synth.WORKLOADS["dense_30L_32x4096"], layers=2, name="dense_30L_32x4096")
    dev = torch.device("cuda:0")
    B, H, dk, dv, N = w.layers, w.heads, w.dk, w.dv, w.n_tokens
    off = w.offsets()
    xs = [synth.torch_layer_inputs(w, layer, dev, want_q=True) for layer in range(B)]
    st = lambda key: torch.stack([x[key] for x in xs]).contiguous()
    q, k, v, a, b = st("q"), st("k"), st("v"), st("alpha"), st("beta")
    out = pic.pic_segment_prefill(q, k, v, a, b, off)
    torch.cuda.synchronize()
    rng = np.random.default_rng(94)
    for layer, h, seg in [(0, 0, 0), (1, 31, 31), (int(rng.integers(B)), int(rng.integers(H)),
                                                    int(rng.integers(w.n_seg)))]:
        sl = slice(int(off[seg]), int(off[seg + 1]))
        f = lambda t: t[layer, sl, h].float().cpu().numpy()[None, :, None]
        ref = oracle.prefill(DENSE, f(q), f(k), f(v), f(a), f(b), [0, sl.stop - sl.start])
        got_o = out["O"][layer, sl, h].float().cpu().numpy()[None, :, None]
        e = _o_err(got_o, ref["O"])
        gpu = {"S0": out["S0"][seg, layer, h].cpu().numpy()[None, None, None],
               "T_hat": out["T_hat"][seg, layer, h].cpu().numpy()[None, None, None],
               "log_scale": out["log_scale"][seg, layer, h].cpu().numpy()[None, None, None]}
        report(f"prefill full length (layer {layer}, head {h}, seg {seg}): output err {e:.3e}")
        assert e <= TOL_BF16
        assert_pair_close(gpu, ref, DENSE, TOL_BF16)
