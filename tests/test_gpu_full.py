"""Parity at the full workload sizes, in the launch configuration the benchmark
times (one build call for all segments, layers and heads; one compose call
per chain batch).

* scalar decay, 32 heads x d=128, 8 x 2048 tokens: every unit against the oracle;
* diagonal gates, 32 heads x d=128, 16 x 4096 tokens: every unit;
* dense GDN, 30 layers x 32 heads x d=128, 32 x 4096 tokens (128K prompt):
  sampled units (the oracle rebuilds them one by one from the same inputs)
  and sampled composed chains; the same for the delta rule with per-channel
  gates (KDA form) at that shape;
* the slow-gate variants, where the carried term T(C2) S(C1) is a sizeable
  part of the state, so composition really exercises T;
* composition-heavy reuse, 30 layers x 32 heads x d=128: a pool of 256
  cached segments (512..8192 tokens) plus 512 fresh 2048-token segments,
  64 requests composing 56-step chains, streamed layer by layer; sampled
  units, chains and chain pairs against the oracle; the same with 8-token
  seam windows on every inner chain entry (final states and seam outputs).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (TOL_BF16, assert_pair_close, lam_err, max_rel_units, report,
                               to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def rho_of(composed_ref, last_S):
    """min over units of ||carried|| / ||state|| with carried = state - S(C_last|0)."""
    a = np.asarray(composed_ref, np.float64).reshape(-1, composed_ref.shape[-2] * composed_ref.shape[-1])
    b = np.asarray(last_S, np.float64).reshape(a.shape)
    return float(np.min(np.linalg.norm(a - b, axis=1) / np.linalg.norm(a, axis=1)))


@pytest.mark.parametrize("name", ["scalar_8x2048", "scalar_8x2048_slow", "diag_16x4096",
                                  "diag_16x4096_slow"])
def test_scalar_diag_full_workload(name):
    import hybrid_caching_amd as pic
    import torch
    w = synth.WORKLOADS[name]
    x = synth.layer_inputs(w)
    dt = torch.bfloat16
    pair = pic.pic_segment_build(w.form, to_dev(x["k"], dt), to_dev(x["v"], dt),
                                 to_dev(x["alpha"]), None, x["offsets"])
    n = w.n_seg
    comp = pic.pic_compose(w.form, pair["log_scale"], None, pair["S0"], [0, n], list(range(n)))
    naive = pic.pic_naive_add(pair["S0"], [0, n], list(range(n)))
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in pair.items()}
    ref = oracle.build(w.form, x["k"], x["v"], x["alpha"], None, x["offsets"])
    assert_pair_close(gpu, ref, w.form, TOL_BF16)
    ref_c = oracle.compose(w.form, ref["lam"], None, ref["S"], [0, n], list(range(n)))
    e = max_rel_units(comp.cpu().numpy(), ref_c)
    rho = rho_of(ref_c[0], ref["S"][-1])
    report(f"{name}: compose err {e:.3e}, rho {rho:.3f}")
    assert e <= TOL_BF16
    if name.endswith("_slow"):
        assert rho >= 0.1
    ref_n = oracle.naive_add(ref["S"], [0, n], list(range(n)))
    assert max_rel_units(naive.cpu().numpy(), ref_n) <= TOL_BF16


def _dense_full(name, layers, samples, chains, precision=0):
    """Build the dense stack on the GPU from device-drawn inputs, then check
    sampled (layer, head, segment) units and sampled composed (layer, head)
    chains against the oracle run on the same input values."""
    import hybrid_caching_amd as pic
    import torch
    w = synth.WORKLOADS[name]
    if layers is not None:
        w = synth.scaled(w, layers=layers, name=w.name)
    B, H, dk, dv, N, n_seg = w.layers, w.heads, w.dk, w.dv, w.n_tokens, w.n_seg
    dev = torch.device("cuda:0")
    k = torch.empty((B, N, H, dk), dtype=torch.bfloat16, device=dev)
    v = torch.empty((B, N, H, dv), dtype=torch.bfloat16, device=dev)
    ashape = (B, N, H, dk) if w.form in synth.PER_CHANNEL_GATES else (B, N, H)
    alpha = torch.empty(ashape, dtype=torch.float32, device=dev)
    beta = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    for layer in range(B):
        x = synth.torch_layer_inputs(w, layer, dev)
        k[layer].copy_(x["k"])
        v[layer].copy_(x["v"])
        alpha[layer].copy_(x["alpha"])
        beta[layer].copy_(x["beta"])
    offsets = w.offsets()
    pair = pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, precision=precision)
    comp = pic.pic_compose(w.form, pair["log_scale"], pair["T_hat"], pair["S0"], [0, n_seg],
                           list(range(n_seg)))
    naive = pic.pic_naive_add(pair["S0"], [0, n_seg], list(range(n_seg)))
    torch.cuda.synchronize()

    def unit_inputs(layer, head, s0, s1):
        sl = slice(int(offsets[s0]), int(offsets[s1]))
        f = lambda t: t[layer, sl, head].float().cpu().numpy()[None, :, None]
        return f(k), f(v), f(alpha), f(beta)

    rng = np.random.default_rng(2024)
    for (layer, head, seg) in samples(rng, B, H, n_seg):
        kk, vv, aa, bb = unit_inputs(layer, head, seg, seg + 1)
        L = kk.shape[1]
        ref = oracle.build(w.form, kk, vv, aa, bb, [0, L])
        gpu = {"S0": pair["S0"][seg, layer, head].cpu().numpy()[None, None, None],
               "T_hat": pair["T_hat"][seg, layer, head].cpu().numpy()[None, None, None],
               "log_scale": pair["log_scale"][seg, layer, head].cpu().numpy()[None, None, None]}
        report(f"{name} precision {precision} unit (layer {layer}, head {head}, seg {seg}):")
        assert_pair_close(gpu, ref, w.form, TOL_BF16)
    for (layer, head) in chains(rng, B, H):
        kk, vv, aa, bb = unit_inputs(layer, head, 0, n_seg)
        offs = offsets
        ref = oracle.build(w.form, kk, vv, aa, bb, offs)
        ref_c = oracle.compose(w.form, ref["lam"], ref["That"], ref["S"], [0, n_seg],
                               list(range(n_seg)))
        got = comp[0, layer, head].cpu().numpy()
        e = max_rel_units(got, ref_c[0, 0, 0])
        rho = rho_of(ref_c[0], ref["S"][-1])
        en = max_rel_units(naive[0, layer, head].cpu().numpy(),
                           oracle.naive_add(ref["S"], [0, n_seg], list(range(n_seg)))[0, 0, 0])
        report(f"{name} precision {precision} chain (layer {layer}, head {head}): "
               f"compose err {e:.3e}, rho {rho:.3f}, "
               f"naive-add err {en:.3e}")
        assert e <= TOL_BF16 and en <= TOL_BF16
        if name.endswith("_slow"):
            assert rho >= 0.1
    return pair


@pytest.mark.parametrize("precision", [0, 1])
def test_dense_full_workload_sampled(precision):
    def samples(rng, B, H, n_seg):
        fixed = [(0, 0, 0), (B - 1, H - 1, n_seg - 1), (B // 2, 7, n_seg // 2)]
        extra = [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(n_seg)))
                 for _ in range(3)]
        return fixed + extra

    def chains(rng, B, H):
        return [(B - 1, 3)]

    _dense_full("dense_30L_32x4096", None, samples, chains, precision)


@pytest.mark.parametrize("precision", [0, 1])
def test_dense_slow_gates_full_length_sampled(precision):
    """Slow gates at the full 32 x 4096 prompt (2 layers): composition of 32
    built segments must match the oracle with a sizeable carried term."""
    def samples(rng, B, H, n_seg):
        return [(1, 5, 3)]

    def chains(rng, B, H):
        return [(0, 0)]

    _dense_full("dense_30L_32x4096_slow", 2, samples, chains, precision)


@pytest.mark.parametrize("precision", [0, 1])
def test_kda_full_workload_sampled(precision):
    """Delta rule with per-channel gates at the dense workload's shape (30
    layers x 32 heads x d=128, 32 x 4096 tokens) in one build call, token by
    token in fp32 and in chunks with fp16 operands: sampled units and one
    composed 32-segment chain against the oracle."""
    def samples(rng, B, H, n_seg):
        fixed = [(0, 0, 0), (B - 1, H - 1, n_seg - 1)]
        return fixed + [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(n_seg)))]

    def chains(rng, B, H):
        return [(B // 2, 11)]

    _dense_full("kda_30L_32x4096", None, samples, chains, precision)


@pytest.mark.parametrize("precision", [0, 1])
def test_kda_slow_gates_full_length_sampled(precision):
    """Slow per-channel gates at the full prompt length (2 layers): the
    composed chain carries a sizeable T(C2) S(C1) term."""
    def samples(rng, B, H, n_seg):
        return [(1, 9, 30)]

    def chains(rng, B, H):
        return [(0, 2)]

    _dense_full("kda_30L_32x4096_slow", 2, samples, chains, precision)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,layers,precision",
                         [("reuse_256x30", None, 0), ("reuse_256x30", None, 1),
                          ("reuse_256x30_slow", 2, 0), ("reuse_256x30_slow", 2, 1)])
def test_reuse_workload_sampled(name, layers, precision):
    """At the base gates the carried term underflows (composition gives the
    last segment's S0 exactly); the slow-gate variant makes it sizeable.
    Precision 1 (fp16 operands) is the build the benchmark times: 768
    variable-length segments of 512..8192 tokens per layer through the
    workspace plan."""
    import hybrid_caching_amd as pic
    import torch
    from oracle import DENSE
    w = synth.WORKLOADS[name]
    if layers is not None:
        w = synth.scaled(w, layers=layers, name=w.name)
    fw = synth.reuse_fresh_workload(w)
    off, idx = synth.reuse_chains(w)
    n_pool, n_fresh = w.n_seg, fw.n_seg
    H, dk, dv = w.heads, w.dk, w.dv
    dev = torch.device("cuda:0")
    P = n_pool + n_fresh
    buf = {"log_scale": torch.empty((P, 1, H), dtype=torch.float32, device=dev),
           "T_hat": torch.empty((P, 1, H, dk, dk), dtype=torch.float32, device=dev),
           "S0": torch.empty((P, 1, H, dk, dv), dtype=torch.float32, device=dev)}
    pool_out = {key: t[:n_pool] for key, t in buf.items()}
    fresh_out = {key: t[n_pool:] for key, t in buf.items()}
    p_off, f_off = w.offsets(), fw.offsets()
    rng = np.random.default_rng(105)
    lens = np.diff(p_off)
    sampled_layers = {0: [], min(17, w.layers - 1): [], w.layers - 1: []}
    for layer in sampled_layers:
        sampled_layers[layer] = {
            "pool": [int(np.argmin(lens)), int(np.argmax(lens)), int(rng.integers(n_pool))],
            "fresh": [int(rng.integers(n_fresh))],
            "heads": [int(rng.integers(H)) for _ in range(3)],
            "reqs": [int(rng.integers(w.extra["n_req"])) for _ in range(2)]}

    def unit(x, offsets, s, h):
        sl = slice(int(offsets[s]), int(offsets[s + 1]))
        f = lambda t: t[sl, h].float().cpu().numpy()[None, :, None]
        return f(x["k"]), f(x["v"]), f(x["alpha"]), f(x["beta"])

    for layer in range(w.layers):
        x = synth.torch_layer_inputs(w, layer, dev)
        pic.pic_segment_build(DENSE, x["k"][None], x["v"][None], x["alpha"][None],
                              x["beta"][None], p_off, out=pool_out, precision=precision)
        y = synth.torch_layer_inputs(fw, layer, dev)
        pic.pic_segment_build(DENSE, y["k"][None], y["v"][None], y["alpha"][None],
                              y["beta"][None], f_off, out=fresh_out, precision=precision)
        want = layer in sampled_layers
        res = pic.pic_compose(DENSE, buf["log_scale"], buf["T_hat"], buf["S0"], off, idx,
                              want_pair=want)
        torch.cuda.synchronize()
        if not want:
            del x, y
            continue
        S_out, lam_out, T_out = res
        smp = sampled_layers[layer]
        h = smp["heads"][0]
        for s in smp["pool"]:
            ref = oracle.build(DENSE, *unit(x, p_off, s, h), [0, int(lens[s])])
            gpu = {key: t[s, 0, h].cpu().numpy()[None, None, None] for key, t in buf.items()}
            report(f"{name} precision {precision} layer {layer}: pool unit {s} "
                   f"({int(lens[s])} tokens), head {h}")
            assert_pair_close(gpu, ref, DENSE, TOL_BF16)
        for s in smp["fresh"]:
            ref = oracle.build(DENSE, *unit(y, f_off, s, h), [0, fw.seg_lens[s]])
            gpu = {key: t[n_pool + s, 0, h].cpu().numpy()[None, None, None]
                   for key, t in buf.items()}
            report(f"{name} precision {precision} layer {layer}: fresh unit {s}, head {h}")
            assert_pair_close(gpu, ref, DENSE, TOL_BF16)
        for r, hh in zip(smp["reqs"], smp["heads"][1:]):
            ids = idx[off[r]:off[r + 1]]
            sub = {key: t[torch.as_tensor(ids.astype(np.int64), device=dev), 0, hh]
                   .cpu().numpy()[:, None, None] for key, t in buf.items()}
            n = len(ids)
            ref_S, ref_l, ref_T = oracle.compose(DENSE, sub["log_scale"], sub["T_hat"],
                                                 sub["S0"], [0, n], list(range(n)),
                                                 want_pair=True)
            e = max_rel_units(S_out[r, 0, hh].cpu().numpy(), ref_S[0, 0, 0])
            eT = max_rel_units(T_out[r, 0, hh].cpu().numpy(), ref_T[0, 0, 0])
            el = lam_err(lam_out[r, 0, hh].cpu().numpy(), ref_l[0, 0, 0])
            rho = rho_of(ref_S[0], sub["S0"][-1])
            report(f"{name} layer {layer}: chain (req {r}, head {hh}, {n} steps): "
                   f"compose err {e:.3e}, chain That err {eT:.3e}, lambda err {el:.1e}, "
                   f"rho {rho:.3f}")
            assert e <= 1e-4 and eT <= 1e-4 and el <= 1e-5
            if name.endswith("_slow"):
                assert rho >= 0.1
        del x, y


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,layers,precision",
                         [("reuse_seam_256x30", 3, 0), ("reuse_seam_256x30", 3, 1),
                          ("reuse_seam_256x30_slow", 2, 0)])
def test_reuse_seam_workload_sampled(name, layers, precision):
    """Reuse with 8-token seam windows on every inner chain entry, at the
    benchmark's per-layer launch size (768 pool and fresh segments, 64 requests
    x 56-entry chains, 32 heads, d = 128), layer by layer; sampled chains
    against the oracle: final state and every seam output."""
    import hybrid_caching_amd as pic
    import torch
    from oracle import DENSE
    w = synth.scaled(synth.WORKLOADS[name], layers=layers, name=synth.WORKLOADS[name].name)
    fw = synth.reuse_fresh_workload(w)
    off, idx = synth.reuse_chains(w)
    seam_off = synth.reuse_seam_offsets(off, w.extra["seam"])
    NS = int(seam_off[-1])
    n_pool, n_fresh = w.n_seg, fw.n_seg
    H, dk, dv = w.heads, w.dk, w.dv
    dev = torch.device("cuda:0")
    P = n_pool + n_fresh
    buf = {"log_scale": torch.empty((P, 1, H), dtype=torch.float32, device=dev),
           "T_hat": torch.empty((P, 1, H, dk, dk), dtype=torch.float32, device=dev),
           "S0": torch.empty((P, 1, H, dk, dv), dtype=torch.float32, device=dev)}
    pool_out = {key: t[:n_pool] for key, t in buf.items()}
    fresh_out = {key: t[n_pool:] for key, t in buf.items()}
    one = synth.scaled(w, layers=1, name=w.name)
    rng = np.random.default_rng(205)
    for layer in range(w.layers):
        x = synth.torch_layer_inputs(w, layer, dev)
        pic.pic_segment_build(DENSE, x["k"][None], x["v"][None], x["alpha"][None],
                              x["beta"][None], w.offsets(), out=pool_out, precision=precision)
        y = synth.torch_layer_inputs(fw, layer, dev)
        pic.pic_segment_build(DENSE, y["k"][None], y["v"][None], y["alpha"][None],
                              y["beta"][None], fw.offsets(), out=fresh_out, precision=precision)
        del x, y
        si = synth.torch_seam_inputs(one, NS, dev, seed_offset=1000 * layer)
        S_out, O = pic.pic_compose_seams(DENSE, buf["log_scale"], buf["T_hat"], buf["S0"], off,
                                         idx, seam_off, si["q"], si["k"], si["v"], si["alpha"],
                                         si["beta"])
        torch.cuda.synchronize()
        for r, hh in [(int(rng.integers(w.extra["n_req"])), int(rng.integers(H))) for _ in range(2)]:
            ids = idx[off[r]:off[r + 1]]
            n = len(ids)
            sub = {key: t[torch.as_tensor(ids.astype(np.int64), device=dev), 0, hh]
                   .cpu().numpy()[:, None, None] for key, t in buf.items()}
            t0, t1 = int(seam_off[off[r]]), int(seam_off[off[r + 1]])
            so = seam_off[off[r]:off[r + 1] + 1] - t0
            tok = lambda key: si[key][0, t0:t1, hh].float().cpu().numpy()[None, :, None]
            ref_S, ref_O = oracle.seam_compose(DENSE, sub["log_scale"], sub["T_hat"], sub["S0"],
                                               [0, n], list(range(n)), so, tok("q"), tok("k"),
                                               tok("v"), tok("alpha"), tok("beta"))
            es = max_rel_units(S_out[r, 0, hh].cpu().numpy(), ref_S[0, 0, 0])
            eo = max_rel_units(O[0, t0:t1, hh].cpu().numpy(), ref_O[0, :, 0])
            rho = rho_of(ref_S[0], sub["S0"][-1])
            report(f"{name} layer {layer}: chain (req {r}, head {hh}, {n} entries, {t1 - t0} "
                   f"seam tokens): state err {es:.3e}, output err {eo:.3e}, rho {rho:.3f}")
            assert es <= 1e-4 and eo <= 1e-4
            if name.endswith("_slow"):
                assert rho >= 0.1


def test_all_segments_empty():
    """n_tokens = 0 with empty segments: identity pairs, zero states."""
    import hybrid_caching_amd as pic
    import torch
    dev = torch.device("cuda:0")
    k = torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16, device=dev)
    v = torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16, device=dev)
    a = torch.zeros((2, 0, 3), dtype=torch.float32, device=dev)
    pair = pic.pic_segment_build(2, k, v, a, None, [0, 0, 0])
    torch.cuda.synchronize()
    assert torch.all(pair["S0"] == 0) and torch.all(pair["log_scale"] == 0)
    eye = torch.eye(64, device=dev).expand_as(pair["T_hat"])
    assert torch.equal(pair["T_hat"], eye)


def test_many_short_segments():
    """Hundreds of segments of 1..200 tokens (ragged, every chunk tail)."""
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 200, size=300)
    offs = np.concatenate([[0], np.cumsum(lens)])
    w = synth.scaled(synth.WORKLOADS["dense_30L_32x4096"], layers=1, heads=2,
                     seg_lens=tuple(int(x) for x in lens), name="dense_many_short")
    x = synth.layer_inputs(w)
    from tests.gpu_helpers import build_both
    gpu, ref = build_both(w.form, x["k"], x["v"], x["alpha"], x["beta"], offs, True)
    assert_pair_close(gpu, ref, w.form, TOL_BF16)
