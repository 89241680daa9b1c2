"""Parity of the HIP convolution warm-up with the fp64 oracle, through the C
ABI (bf16 and fp32 inputs, widths 1-4, full / partial / absent history), and
the whole method on the GPU: warm-up windows computed here and run by the seam
compose after pairs built on the segment tails, against the oracle's
recurrence over the whole prompt's conv outputs.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import DENSE
from tests.gpu_helpers import TOL_F32, max_rel_units, report, to_dev
from tests.test_oracle_conv_pins import conv_full

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("W,dc", [(4, 128), (4, 16), (2, 64), (1, 32)])
def test_conv_warmup_matches_oracle(bf16, W, dc):
    import hybrid_caching_amd as pic
    import torch
    rng = np.random.default_rng(W * 100 + dc + bf16)
    B, H, N = 2, 3, 90
    x = rng.standard_normal((B, N, H, dc)).astype(np.float32)
    if bf16:
        x = synth.bf16_round(x)
    w = (rng.standard_normal((H, dc, W)) / W).astype(np.float32)
    n_warm = max(W - 1, 1)
    heads = [0, 10, 11, 40, 87 - n_warm + 3]
    heads = [min(h, N - n_warm) for h in heads]
    hist_end = [0, 10, 11, 38, heads[4]]
    hist_len = [0, min(W - 1, 10), min(W - 1, 1), min(W - 1, 38), W - 1]
    y = pic.pic_conv_warmup(to_dev(w), to_dev(x, torch.bfloat16 if bf16 else torch.float32),
                            heads, hist_end, hist_len, n_warm)
    torch.cuda.synchronize()
    want = oracle.conv_warmup(w, x, hist_end, hist_len, heads, n_warm)
    e = max_rel_units(y.float().cpu().numpy(), want)
    report(f"W {W} dc {dc} bf16 {bf16}: err {e:.3e}")
    assert e <= (4e-3 if bf16 else TOL_F32)


@pytest.mark.parametrize("W,n_warm", [(4, 3), (4, 7), (4, 1), (4, 13), (4, 14), (9, 8), (16, 15),
                                     (5, 12)])
def test_conv_warmup_many_blocks(W, n_warm):
    """A launch of several channel-item blocks (32 heads x 128 channels = 4
    blocks of 256 items) and many 32-row blocks (2 layers x 20 entries x
    n_warm rows), widths up to the header's limit of 16 and windows longer
    than W - 1, with full, partial and absent history.  Width 4 runs the
    window-in-registers kernel up to n_warm = 13 (3 + 13 taps) and the general
    one beyond."""
    import hybrid_caching_amd as pic
    import torch
    rng = np.random.default_rng(1000 + 31 * W + n_warm)
    B, H, dc, N, n = 2, 32, 128, 700, 20
    x = synth.bf16_round(rng.standard_normal((B, N, H, dc)).astype(np.float32))
    w = (rng.standard_normal((H, dc, W)) / W).astype(np.float32)
    starts = sorted(rng.choice(np.arange(0, N - n_warm), size=n, replace=False).tolist())
    hist_end = [int(s) for s in starts]
    hist_len = [min(W - 1, int(s), int(rng.integers(0, W))) for s in starts]
    hist_len[0] = min(W - 1, starts[0])
    y = pic.pic_conv_warmup(to_dev(w), to_dev(x, torch.bfloat16), starts, hist_end, hist_len,
                            n_warm)
    torch.cuda.synchronize()
    assert y.shape == (B, n * n_warm, H, dc)
    assert B * n * n_warm > 32 and H * dc // 4 > 256
    want = oracle.conv_warmup(w, x, hist_end, hist_len, starts, n_warm)
    e = max_rel_units(y.float().cpu().numpy(), want)
    report(f"many blocks W {W} n_warm {n_warm}: err {e:.3e}")
    assert e <= 4e-3


def test_conv_warmup_through_seams_equals_the_prompt():
    """The whole method on the GPU, fp32: pairs of each segment's tokens
    after its window (conv on the segment alone), the windows recomputed by
    the warm-up kernel with the previous segment's raw tail, seam compose:
    the recurrence over the whole prompt's conv outputs."""
    import hybrid_caching_amd as pic
    import torch
    W, B, H, dk, dv = 4, 2, 2, 64, 64
    cuts = [0, 70, 151, 300]
    n = len(cuts) - 1
    N = cuts[-1]
    rng = np.random.default_rng(17)
    xk = rng.standard_normal((B, N, H, dk)).astype(np.float32)
    xv = rng.standard_normal((B, N, H, dv)).astype(np.float32)
    xq = rng.standard_normal((B, N, H, dk)).astype(np.float32)
    wk = (rng.standard_normal((H, dk, W)) / (8 * W)).astype(np.float32)
    wv = (rng.standard_normal((H, dv, W)) / W).astype(np.float32)
    wq = (rng.standard_normal((H, dk, W)) / W).astype(np.float32)
    a = rng.uniform(0.99, 1.0, size=(B, N, H)).astype(np.float32)
    b = rng.uniform(0.0, 0.2, size=(B, N, H)).astype(np.float32)
    tails_k, tails_v, al, be, rest = [], [], [], [], [0]
    for s in range(n):
        seg = slice(cuts[s], cuts[s + 1])
        tails_k.append(conv_full(wk, xk[:, seg])[:, W - 1:])
        tails_v.append(conv_full(wv, xv[:, seg])[:, W - 1:])
        al.append(a[:, cuts[s] + W - 1:cuts[s + 1]])
        be.append(b[:, cuts[s] + W - 1:cuts[s + 1]])
        rest.append(rest[-1] + cuts[s + 1] - cuts[s] - (W - 1))
    f32 = lambda z: to_dev(np.ascontiguousarray(np.concatenate(z, 1), dtype=np.float32))
    pair = pic.pic_segment_build(DENSE, f32(tails_k), f32(tails_v), f32(al), f32(be), rest)
    starts = cuts[:-1]
    hist = [min(W - 1, s) for s in starts]
    dev_x = lambda z: to_dev(z)
    sk = pic.pic_conv_warmup(to_dev(wk), dev_x(xk), starts, starts, hist, W - 1)
    sv = pic.pic_conv_warmup(to_dev(wv), dev_x(xv), starts, starts, hist, W - 1)
    sq = pic.pic_conv_warmup(to_dev(wq), dev_x(xq), starts, starts, hist, W - 1)
    idx = np.concatenate([np.arange(s, s + W - 1) for s in starts])
    sa = to_dev(np.ascontiguousarray(a[:, idx]))
    sb = to_dev(np.ascontiguousarray(b[:, idx]))
    seam_off = [e * (W - 1) for e in range(n + 1)]
    S_out, O = pic.pic_compose_seams(DENSE, pair["log_scale"], pair["T_hat"], pair["S0"], [0, n],
                                     list(range(n)), seam_off, sq, sk, sv, sa, sb)
    torch.cuda.synchronize()
    want = oracle.recurrence(DENSE, conv_full(wk, xk), conv_full(wv, xv), a, b)
    e = max_rel_units(S_out.cpu().numpy()[0], want)
    report(f"warm-up windows through seams: state err {e:.3e}")
    assert e <= TOL_F32
