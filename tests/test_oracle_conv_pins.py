"""Pins of the oracle's convolution warm-up (a short causal depthwise
convolution of width W in front of the linear layer).  [xix.ai HYPIC article
(French), paragraph on linear layers: variants with a short convolution need
the convolution state warmed up.]

Reading: the conv output of token t depends on raw inputs t-W+1 .. t, so only a
segment's first W-1 tokens see the previous segment; they stay out of the
cached pair and are recomputed on reuse with the real history, then run
through the state as a seam window.  The pins compare with numpy's convolve
over the whole prompt, the independent prefill, and the recurrence over the
whole prompt's conv outputs.
"""
import numpy as np
import pytest

import oracle
from oracle import DENSE, SCALAR
from tests.conftest import rel_fro


def conv_full(w, x):
    """Causal depthwise conv over the token axis by np.convolve: x [B, N, H, dc],
    w [H, dc, W] -> y [B, N, H, dc]."""
    B, N, H, dc = x.shape
    y = np.zeros((B, N, H, dc))
    for b in range(B):
        for h in range(H):
            for c in range(dc):
                y[b, :, h, c] = np.convolve(x[b, :, h, c], w[h, c])[:N]
    return y


def case(B, H, dc, W, cuts, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, cuts[-1], H, dc))
    w = rng.standard_normal((H, dc, W)) / W
    return w, x


@pytest.mark.parametrize("W", [2, 4])
def test_warmup_equals_the_whole_prompt_conv(W):
    cuts = [0, 9, 12, 30, 41]
    w, x = case(2, 3, 5, W, cuts, seed=W)
    y_full = conv_full(w, x)
    starts = cuts[:-1]
    hist_len = [min(W - 1, s) for s in starts]
    y = oracle.conv_warmup(w, x, starts, hist_len, starts, W - 1)
    for e, s in enumerate(starts):
        for t in range(W - 1):
            assert np.abs(y[:, e * (W - 1) + t] - y_full[:, s + t]).max() <= 1e-12


def test_zero_history_is_the_independent_prefill():
    W = 4
    cuts = [0, 10, 25]
    w, x = case(1, 2, 3, W, cuts, seed=5)
    y = oracle.conv_warmup(w, x, [0, 10], [0, 0], [0, 10], W - 1)
    alone = conv_full(w, x[:, 10:25])
    assert np.abs(y[:, 3:6] - alone[:, :3]).max() <= 1e-12
    assert np.abs(y[:, 0:3] - conv_full(w, x[:, :10])[:, :3]).max() <= 1e-12


def test_width_one_is_a_channel_scaling():
    w, x = case(1, 2, 4, 1, [0, 6], seed=6)
    y = oracle.conv_warmup(w, x, [3], [0], [3], 1)
    assert np.abs(y[:, 0] - w[None, :, :, 0] * x[:, 3]).max() <= 1e-15


def test_tokens_past_the_window_need_no_history():
    """The reading's premise: from token W-1 on, a segment's conv outputs
    computed alone equal those computed in the prompt."""
    W = 4
    cuts = [0, 20, 45]
    w, x = case(1, 2, 3, W, cuts, seed=7)
    y_full = conv_full(w, x)
    alone = conv_full(w, x[:, 20:45])
    assert np.abs(alone[:, W - 1:] - y_full[:, 20 + W - 1:45]).max() <= 1e-12
    assert np.abs(alone[:, :W - 1] - y_full[:, 20:20 + W - 1]).max() > 1e-3


@pytest.mark.parametrize("form", [DENSE, SCALAR])
def test_warmup_windows_compose_into_the_prompt_recurrence(form):
    """The whole method: pairs built on each segment's tokens after its
    window (conv computed on the segment alone), windows recomputed with the
    previous segment's raw tail and run as seams, composed: the recurrence over
    the whole prompt's conv outputs."""
    W, B, H, dk, dv = 4, 1, 2, 6, 5
    cuts = [0, 13, 30, 47]
    n = len(cuts) - 1
    rng = np.random.default_rng(11)
    N = cuts[-1]
    xk = rng.standard_normal((B, N, H, dk))
    xv = rng.standard_normal((B, N, H, dv))
    xq = rng.standard_normal((B, N, H, dk))
    wk = rng.standard_normal((H, dk, W)) / (2 * W)
    wv = rng.standard_normal((H, dv, W)) / W
    wq = rng.standard_normal((H, dk, W)) / W
    a = rng.uniform(0.9, 1.0, size=(B, N, H))
    b = rng.uniform(0.0, 0.3, size=(B, N, H)) if form == DENSE else None
    # pairs: each segment alone, tokens from W-1 on
    ks, vs, als, bes, rest_cuts = [], [], [], [], [0]
    for s in range(n):
        seg = slice(cuts[s], cuts[s + 1])
        ks.append(conv_full(wk, xk[:, seg])[:, W - 1:])
        vs.append(conv_full(wv, xv[:, seg])[:, W - 1:])
        als.append(a[:, cuts[s] + W - 1:cuts[s + 1]])
        if b is not None:
            bes.append(b[:, cuts[s] + W - 1:cuts[s + 1]])
        rest_cuts.append(rest_cuts[-1] + (cuts[s + 1] - cuts[s] - (W - 1)))
    pairs = oracle.build(form, np.concatenate(ks, 1), np.concatenate(vs, 1),
                         np.concatenate(als, 1), np.concatenate(bes, 1) if b is not None else None,
                         rest_cuts)
    # windows: the first W-1 tokens of every segment with the prompt's history
    starts = cuts[:-1]
    hist = [min(W - 1, s) for s in starts]
    sk = oracle.conv_warmup(wk, xk, starts, hist, starts, W - 1)
    sv = oracle.conv_warmup(wv, xv, starts, hist, starts, W - 1)
    sq = oracle.conv_warmup(wq, xq, starts, hist, starts, W - 1)
    idx = np.concatenate([np.arange(s, s + W - 1) for s in starts])
    sa = a[:, idx]
    sb = b[:, idx] if b is not None else None
    seam_off = [e * (W - 1) for e in range(n + 1)]
    S_out, O = oracle.seam_compose(form, pairs["lam"], pairs.get("That"), pairs["S"], [0, n],
                                   list(range(n)), seam_off, sq, sk, sv, sa, sb)
    k_all, v_all = conv_full(wk, xk), conv_full(wv, xv)
    want = oracle.recurrence(form, k_all, v_all, a, b)
    assert rel_fro(S_out[0], want) <= 1e-11
    # and without the warm-up (windows computed with no history) it is not
    sk0 = oracle.conv_warmup(wk, xk, starts, [0] * n, starts, W - 1)
    sv0 = oracle.conv_warmup(wv, xv, starts, [0] * n, starts, W - 1)
    S_bad, _ = oracle.seam_compose(form, pairs["lam"], pairs.get("That"), pairs["S"], [0, n],
                                   list(range(n)), seam_off, sq, sk0, sv0, sa, sb)
    assert rel_fro(S_bad[0], want) > 1e-3
