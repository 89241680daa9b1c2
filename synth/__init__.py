"""Seeded synthetic inputs for the segment transform (build / compose / naive add).

This module holds only random draws, rounding to storage precision and the
workload shapes.  It contains none of the method's arithmetic.  Both the fp64
oracle (``oracle/``) and the HIP path (``hybrid_caching_amd``) are fed from
here, so the two see bit-identical inputs.

The shapes mimic the workloads of the HYPIC articles: prompts assembled from
tens to hundreds of independent segments, each usually longer than 512
tokens, contexts up to ~128K tokens, and a Qwen3.5-35B-A3B-like hybrid model
with 30 linear-attention layers of 32 heads, head dim 128 (about 2 MB of
recurrent state per layer).  [xix.ai HYPIC article (French), paragraphs on
workloads and on the seam window; remio.ai (Japanese), section on why prefix
caching falls short for RAG and agents.]  The articles evaluate on public QA
and summarisation datasets and a production RAG trace; none of those is
used: these seeded synthetic draws stand in for them.

Value distributions are not on the pages; they are stated per workload below.
Each (layer, segment) block has its own generator,
``np.random.default_rng(SeedSequence([seed, layer, seg_id, stream]))`` with
stream 0 = k, 1 = v, 2 = q, 3 = alpha, 4 = beta, so any unit can be rebuilt
alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

SCALAR, DIAG, DENSE, KDA = 0, 1, 2, 3
FORM_NAMES = {SCALAR: "scalar", DIAG: "diag", DENSE: "dense", KDA: "kda"}
PER_CHANNEL_GATES = (DIAG, KDA)  # forms with one gate per key channel

# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); return fp32
    arrays holding exactly those bfloat16 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return rounded.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bfloat16 encodings of fp32 values that are exact bfloat16."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (x.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    form: int
    layers: int
    heads: int
    dk: int
    dv: int
    seg_lens: tuple          # token count of each segment of the prompt
    seed: int
    qkv_bf16: bool           # k/v/q stored as bfloat16 (else fp32)
    k_norm: str              # "l2" (unit rows, fp32 before rounding) or "scaled" (1/sqrt(dk))
    v_scale: float           # v ~ N(0, v_scale^2)
    alpha: tuple             # ("uniform", lo, hi) or ("sigmoid_normal", mu, sigma)
    beta: tuple              # ("uniform", lo, hi) or ("one",)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_seg(self):
        return len(self.seg_lens)

    @property
    def n_tokens(self):
        return int(sum(self.seg_lens))

    def offsets(self):
        return np.concatenate([[0], np.cumsum(self.seg_lens)]).astype(np.int64)


WORKLOADS = {
    # tiny dense gated delta, fp32 end to end
    "tiny_dense": Workload("tiny_dense", DENSE, 1, 2, 16, 16, (64, 64), 101, False, "l2", 1.0,
                           ("uniform", 0.9, 1.0), ("uniform", 0.0, 1.0)),
    # scalar decay (RetNet / Mamba2-like): 32 heads, d=128, 8 x 2048 tokens
    "scalar_8x2048": Workload("scalar_8x2048", SCALAR, 1, 32, 128, 128, (2048,) * 8, 102, True,
                              "scaled", 1.0 / np.sqrt(128.0), ("uniform", 0.95, 1.0), ("one",)),
    # diagonal gates (GLA-like): 32 heads, d=128, 16 x 4096 tokens
    "diag_16x4096": Workload("diag_16x4096", DIAG, 1, 32, 128, 128, (4096,) * 16, 103, True,
                             "scaled", 1.0 / np.sqrt(128.0), ("sigmoid_normal", 3.0, 1.0),
                             ("one",)),
    # dense gated delta, 30 linear layers x 32 heads x d=128, 128K tokens as 32 x 4096
    "dense_30L_32x4096": Workload("dense_30L_32x4096", DENSE, 30, 32, 128, 128, (4096,) * 32,
                                  104, True, "l2", 1.0, ("uniform", 0.9, 1.0),
                                  ("uniform", 0.0, 1.0)),
    # delta rule with per-channel gates (KDA form), the same model shape and
    # prompt as the dense workload: per-channel gates as in the diagonal
    # workload, erase strengths as in the dense one
    "kda_30L_32x4096": Workload("kda_30L_32x4096", KDA, 30, 32, 128, 128, (4096,) * 32, 106,
                                True, "l2", 1.0, ("sigmoid_normal", 3.0, 1.0),
                                ("uniform", 0.0, 1.0)),
}

# Few-unit launches: one long segment of one layer, 32 heads (32 units on a
# 256-CU part), the case the split build is for
WORKLOADS["few_dense_1x65536"] = Workload("few_dense_1x65536", DENSE, 1, 32, 128, 128, (65536,),
                                          107, True, "l2", 1.0, ("uniform", 0.9, 1.0),
                                          ("uniform", 0.0, 1.0), extra={"split_demo": True})
WORKLOADS["few_scalar_1x65536"] = Workload("few_scalar_1x65536", SCALAR, 1, 32, 128, 128,
                                           (65536,), 108, True, "scaled", 1.0 / np.sqrt(128.0),
                                           ("uniform", 0.95, 1.0), ("one",),
                                           extra={"split_demo": True})

# Variants with slow gates, so that the T(C2) S(C1) term is a sizeable part of
# the composed state and composition checks really exercise T (at the base
# gate values the incoming state decays below fp32 range across a segment).
WORKLOADS["scalar_8x2048_slow"] = replace(WORKLOADS["scalar_8x2048"], name="scalar_8x2048_slow",
                                          alpha=("uniform", 0.9995, 1.0))
WORKLOADS["diag_16x4096_slow"] = replace(WORKLOADS["diag_16x4096"], name="diag_16x4096_slow",
                                         alpha=("sigmoid_normal", 9.0, 1.0))
WORKLOADS["dense_30L_32x4096_slow"] = replace(WORKLOADS["dense_30L_32x4096"],
                                              name="dense_30L_32x4096_slow",
                                              alpha=("uniform", 0.9995, 1.0),
                                              beta=("uniform", 0.0, 0.02))
WORKLOADS["kda_30L_32x4096_slow"] = replace(WORKLOADS["kda_30L_32x4096"],
                                            name="kda_30L_32x4096_slow",
                                            alpha=("sigmoid_normal", 9.0, 1.0),
                                            beta=("uniform", 0.0, 0.02))


def reuse_pool_lengths(seed: int = 105, pool_size: int = 256, lo: int = 512,
                       hi: int = 8192) -> tuple:
    """Token counts of the cached pool of the reuse workload, ~ U{lo..hi}."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7777]))
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=pool_size))


# composition-heavy reuse: a pool of 256 cached dense segments (lengths
# U{512..8192}) for 30 layers x 32 heads x d=128; 64 requests, each composing
# 48 distinct pool segments (Zipf s = 1.1) and 8 fresh 2048-token segments
# in a shuffled order.  seg_lens are the pool's; the fresh segments are
# drawn by ``reuse_fresh_workload``.
REUSE = {"pool_size": 256, "n_req": 64, "pool_per_req": 48, "fresh_per_req": 8,
         "fresh_len": 2048, "zipf_s": 1.1}
WORKLOADS["reuse_256x30"] = Workload("reuse_256x30", DENSE, 30, 32, 128, 128,
                                     reuse_pool_lengths(), 105, True, "l2", 1.0,
                                     ("uniform", 0.9, 1.0), ("uniform", 0.0, 1.0),
                                     extra=dict(REUSE))


WORKLOADS["reuse_256x30_slow"] = replace(WORKLOADS["reuse_256x30"], name="reuse_256x30_slow",
                                         alpha=("uniform", 0.9995, 1.0),
                                         beta=("uniform", 0.0, 0.02))


# the same reuse with seam windows: every chain entry after a request's first
# starts with an 8-token window that is not in its cached pair and is run from
# the running state on reuse (the pages' default w = 8)
WORKLOADS["reuse_seam_256x30"] = replace(WORKLOADS["reuse_256x30"], name="reuse_seam_256x30",
                                         extra=dict(REUSE, seam=8))


WORKLOADS["reuse_seam_256x30_slow"] = replace(WORKLOADS["reuse_256x30_slow"],
                                              name="reuse_seam_256x30_slow",
                                              extra=dict(REUSE, seam=8))


def reuse_seam_offsets(chain_offsets, w: int) -> np.ndarray:
    """Seam offsets of a reuse call: w tokens for every chain entry except
    the first of each request.  Returns int64 [chain_total + 1]."""
    off = np.asarray(chain_offsets, dtype=np.int64)
    lens = np.full(int(off[-1]), w, dtype=np.int64)
    lens[off[:-1][off[:-1] < off[1:]]] = 0
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def torch_seam_inputs(w: Workload, n_seam: int, device, seed_offset: int = 0):
    """Seam tokens of a reuse call for all layers, drawn on the device with
    the workload's distributions: q, k, v [layers, n_seam, heads, d] (k rows
    L2-normalised as configured, q ~ N(0, 1/dk)), alpha, beta fp32."""
    import torch

    B, H, dk, dv = w.layers, w.heads, w.dk, w.dv
    sdt = torch.bfloat16 if w.qkv_bf16 else torch.float32
    out = {"q": torch.empty((B, n_seam, H, dk), dtype=sdt, device=device),
           "k": torch.empty((B, n_seam, H, dk), dtype=sdt, device=device),
           "v": torch.empty((B, n_seam, H, dv), dtype=sdt, device=device),
           "alpha": torch.empty((B, n_seam, H, dk) if w.form in PER_CHANNEL_GATES
                                else (B, n_seam, H),
                                dtype=torch.float32, device=device),
           "beta": torch.empty((B, n_seam, H), dtype=torch.float32, device=device)}
    seam_w = replace(w, seg_lens=(int(n_seam),))
    for layer in range(B):
        x = torch_layer_inputs(seam_w, layer, device, seed_offset=seed_offset + 7)
        out["k"][layer].copy_(x["k"])
        out["v"][layer].copy_(x["v"])
        out["alpha"][layer].copy_(x["alpha"])
        if x["beta"] is not None:
            out["beta"][layer].copy_(x["beta"])
        del x
        g = torch.Generator(device=device)
        g.manual_seed(int(w.seed) * 1000003 + layer * 7919 + seed_offset + 11)
        out["q"][layer].copy_((torch.randn((n_seam, H, dk), generator=g, device=device)
                               * (1.0 / np.sqrt(dk))).to(sdt))
    return out


def reuse_fresh_workload(w: Workload) -> Workload:
    """The fresh segments of a reuse workload (n_req x fresh_per_req of
    fresh_len tokens), same distributions, its own seed stream."""
    e = w.extra
    return replace(w, name=w.name + "_fresh", seed=w.seed + 50,
                   seg_lens=(e["fresh_len"],) * (e["n_req"] * e["fresh_per_req"]))


def reuse_chains(w: Workload):
    """Chains of the reuse workload: pool ids 0..pool_size-1, fresh ids
    pool_size + fresh_per_req * r + j.  Returns (offsets, idx)."""
    e = w.extra
    return zipf_chains(e["pool_size"], e["n_req"], e["pool_per_req"], e["zipf_s"], w.seed,
                       fresh_per_req=e["fresh_per_req"], fresh_base=e["pool_size"])


def scaled(w: Workload, *, layers=None, heads=None, seg_lens=None, dk=None, dv=None,
           name=None) -> Workload:
    """A smaller copy of a workload with the same distributions."""
    return replace(w, name=name or (w.name + "_small"),
                   layers=layers if layers is not None else w.layers,
                   heads=heads if heads is not None else w.heads,
                   seg_lens=tuple(seg_lens) if seg_lens is not None else w.seg_lens,
                   dk=dk if dk is not None else w.dk, dv=dv if dv is not None else w.dv)


# --------------------------------------------------------------------------
# per-(layer, segment) draws (numpy)
# --------------------------------------------------------------------------

STREAM_K, STREAM_V, STREAM_Q, STREAM_ALPHA, STREAM_BETA = 0, 1, 2, 3, 4


def _rng(w: Workload, layer: int, seg_id: int, stream: int):
    return np.random.default_rng(np.random.SeedSequence([w.seed, layer, seg_id, stream]))


def _store(w: Workload, x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    return bf16_round(x) if w.qkv_bf16 else x


def segment_inputs(w: Workload, layer: int, seg_id: int, L: int, want_q: bool = False):
    """Inputs of one segment of one layer, all heads: k [L,H,dk], v [L,H,dv],
    alpha [L,H] (diag, KDA: [L,H,dk]), beta [L,H] (None when beta = 1), q (opt).
    k, v, q are fp32 arrays holding the stored (bf16 or fp32) values."""
    H, dk, dv = w.heads, w.dk, w.dv
    x = _rng(w, layer, seg_id, STREAM_K).standard_normal((L, H, dk), dtype=np.float32)
    if w.k_norm == "l2":
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
        x = x / np.maximum(n, np.float32(1e-30))
    else:
        x = x * np.float32(1.0 / np.sqrt(dk))
    k = _store(w, x)
    v = _store(w, _rng(w, layer, seg_id, STREAM_V).standard_normal((L, H, dv), dtype=np.float32)
               * np.float32(w.v_scale))
    ra = _rng(w, layer, seg_id, STREAM_ALPHA)
    ashape = (L, H, dk) if w.form in PER_CHANNEL_GATES else (L, H)
    if w.alpha[0] == "uniform":
        alpha = ra.uniform(w.alpha[1], w.alpha[2], size=ashape).astype(np.float32)
    else:
        z = ra.normal(w.alpha[1], w.alpha[2], size=ashape)
        alpha = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    # keep the gate inside (0, 1]: a draw that rounds to exactly 0 is not a gate
    alpha = np.clip(alpha, np.float32(1e-30), np.float32(1.0))
    beta = None
    if w.beta[0] == "uniform":
        beta = _rng(w, layer, seg_id, STREAM_BETA).uniform(
            w.beta[1], w.beta[2], size=(L, H)).astype(np.float32)
    out = {"k": k, "v": v, "alpha": alpha, "beta": beta}
    if want_q:
        out["q"] = _store(w, _rng(w, layer, seg_id, STREAM_Q).standard_normal((L, H, dk),
                                                                                dtype=np.float32))
    return out


def layer_inputs(w: Workload, layers=None, seg_ids=None, want_q: bool = False):
    """Inputs for the given layers (default all), segments concatenated along
    the token axis: k [B,N,H,dk], v [B,N,H,dv], alpha [B,N,H(,dk)], beta [B,N,H]
    or None, plus offsets [n_seg+1]."""
    layers = list(range(w.layers)) if layers is None else list(layers)
    seg_ids = list(range(w.n_seg)) if seg_ids is None else list(seg_ids)
    ks, vs, als, bes, qs = [], [], [], [], []
    for b in layers:
        parts = [segment_inputs(w, b, s, w.seg_lens[s], want_q) for s in seg_ids]
        ks.append(np.concatenate([p["k"] for p in parts]))
        vs.append(np.concatenate([p["v"] for p in parts]))
        als.append(np.concatenate([p["alpha"] for p in parts]))
        if parts[0]["beta"] is not None:
            bes.append(np.concatenate([p["beta"] for p in parts]))
        if want_q:
            qs.append(np.concatenate([p["q"] for p in parts]))
    lens = [w.seg_lens[s] for s in seg_ids]
    out = {"k": np.stack(ks), "v": np.stack(vs), "alpha": np.stack(als),
           "beta": np.stack(bes) if bes else None,
           "offsets": np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)}
    if want_q:
        out["q"] = np.stack(qs)
    return out


# --------------------------------------------------------------------------
# device-side draws (torch), for the full-size workloads
# --------------------------------------------------------------------------


def torch_layer_inputs(w: Workload, layer: int, device, seed_offset: int = 0,
                       want_q: bool = False):
    """Draw one layer's inputs directly on a device with torch's generator.

    Same distributions and layout as ``layer_inputs`` (different random
    stream).  Returns torch tensors k/v (bf16 or fp32), alpha, beta (fp32 or
    None) for all segments of the layer concatenated along tokens, and with
    ``want_q`` queries q ~ N(0, 1/dk) from a stream of their own (the other
    draws do not change)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(w.seed) * 1000003 + int(layer) * 7919 + int(seed_offset))
    N, H, dk, dv = w.n_tokens, w.heads, w.dk, w.dv
    sdt = torch.bfloat16 if w.qkv_bf16 else torch.float32
    x = torch.randn((N, H, dk), generator=g, device=device, dtype=torch.float32)
    if w.k_norm == "l2":
        x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    else:
        x = x * (1.0 / np.sqrt(dk))
    k = x.to(sdt)
    del x
    v = (torch.randn((N, H, dv), generator=g, device=device, dtype=torch.float32)
         * float(w.v_scale)).to(sdt)
    ashape = (N, H, dk) if w.form in PER_CHANNEL_GATES else (N, H)
    if w.alpha[0] == "uniform":
        alpha = torch.rand(ashape, generator=g, device=device, dtype=torch.float32)
        alpha = alpha * (w.alpha[2] - w.alpha[1]) + w.alpha[1]
    else:
        z = torch.randn(ashape, generator=g, device=device, dtype=torch.float32)
        alpha = torch.sigmoid(z * w.alpha[2] + w.alpha[1])
    alpha = alpha.clamp(1e-30, 1.0)
    beta = None
    if w.beta[0] == "uniform":
        beta = torch.rand((N, H), generator=g, device=device, dtype=torch.float32)
        beta = beta * (w.beta[2] - w.beta[1]) + w.beta[1]
    out = {"k": k, "v": v, "alpha": alpha, "beta": beta}
    if want_q:
        out["q"] = torch_layer_queries(w, layer, device, seed_offset)
    return out


def torch_layer_queries(w: Workload, layer: int, device, seed_offset: int = 0):
    """The queries of one layer, q ~ N(0, 1/dk) on the device, from a stream of
    their own (the ``q`` of ``torch_layer_inputs(..., want_q=True)``)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(w.seed) * 1000003 + int(layer) * 7919 + int(seed_offset) + 104729)
    sdt = torch.bfloat16 if w.qkv_bf16 else torch.float32
    return (torch.randn((w.n_tokens, w.heads, w.dk), generator=g, device=device,
                        dtype=torch.float32) * (1.0 / np.sqrt(w.dk))).to(sdt)


# --------------------------------------------------------------------------
# chains of cached segments
# --------------------------------------------------------------------------


def zipf_chains(pool_size: int, n_req: int, per_req: int, s: float, seed: int,
                fresh_per_req: int = 0, fresh_base: int = None):
    """Chains of distinct pool ids per request, drawn without replacement with
    P(rank) ~ rank^-s over a seeded rank->id permutation; each request's
    ``fresh_per_req`` fresh ids (fresh_base + fresh_per_req*r + j) are appended
    and the whole chain is shuffled.  Returns (offsets int64 [R+1], idx int32)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 9999]))
    perm = rng.permutation(pool_size)
    p = np.arange(1, pool_size + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    chains = []
    for r in range(n_req):
        ranks = rng.choice(pool_size, size=per_req, replace=False, p=p)
        ids = list(perm[ranks])
        if fresh_per_req:
            ids += [fresh_base + fresh_per_req * r + j for j in range(fresh_per_req)]
        ids = np.array(ids, dtype=np.int64)
        rng.shuffle(ids)
        chains.append(ids)
    off = np.concatenate([[0], np.cumsum([len(c) for c in chains])]).astype(np.int64)
    idx = np.concatenate(chains).astype(np.int32) if chains else np.zeros(0, np.int32)
    return off, idx


def random_state(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """A seeded fp32 N(0, scale^2) state tensor (e.g. an incoming S_in)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4242]))
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)
