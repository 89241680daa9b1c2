#!/usr/bin/env python3
"""Throughput of the segment transform on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  plan + build the cached pair of every (segment, layer, head)  [dense GDN form]
  + compose the segments in prompt order into one running state per layer
  + the naive-add ablation over the same chain.
Default workload: a Qwen3.5-35B-A3B-like linear-attention stack -- 30 linear
layers x 32 heads, d_k = d_v = 128, fp32 state (2 MiB per layer), bf16 k/v
with L2-normalised keys, beta ~ U(0,1), alpha ~ U(0.9,1) -- and a 128K-token
prompt made of 32 segments of 4096 tokens, all built in one call.

Prints one JSON line.  ``value`` is prompt tokens per second of the whole
step (inputs resident in HBM before timing starts).  Per-kernel durations are
measured with HIP events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "segment build tokens/s + state composes/s (dense delta, H=32, d=128); % roofline"
CHUNK = 64
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "hybrid_caching_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# the source files each timed kernel is compiled from
KERNEL_SOURCES = {
    "build_dense_ws_kernel": ["k_build_dense_ws.hip", "mfma_util.hpp", "pic_internal.hpp",
                              "stage_util.hpp"],
    "build_dense_h16_kernel": ["k_build_dense_h16.hip", "mfma_util.hpp", "pic_internal.hpp"],
    "build_scalar_pipe_kernel": ["k_build_sd_pipe.hip", "mfma_util.hpp", "pic_internal.hpp"],
    "build_diag_pipe_kernel": ["k_build_sd_pipe.hip", "mfma_util.hpp", "pic_internal.hpp"],
    "compose_dense_full_kernel": ["k_compose.hip", "mfma_util.hpp", "pic_internal.hpp"],
    "compose_seam_kernel": ["k_compose_seam.hip", "mfma_util.hpp", "pic_internal.hpp"],
    "build_kda_kernel": ["k_build_kda.hip", "pic_internal.hpp"],
    "build_kda_chunk_kernel": ["k_build_kda_chunk.hip", "mfma_util.hpp", "pic_internal.hpp"],
    "rerotate_kernel": ["k_rerotate.hip", "pic_internal.hpp"],
    "conv_warmup_kernel": ["k_conv_warmup.hip", "pic_internal.hpp"],
    "conv_warmup_w4_kernel": ["k_conv_warmup.hip", "pic_internal.hpp"],
    "dense_fp16_kernel": ["k_dense_fp16.hip", "mfma_util.hpp", "pic_internal.hpp"],
}
PEAK_FP32_VALU_TFLOPS = 78.6  # MI355X fp32 vector FMA rate without packed instructions


def source_digest(kernel: str) -> str:
    """sha256 (first 16 hex digits) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload`, read from the committed
    hardware-counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a plain copy of known size).  None when there is no such
    summary or the kernel's sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.hbm_counters.md")
    try:
        with open(path) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    if fields.get("sources_sha256") != source_digest(kernel):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, dev, nbytes: int) -> None:
    """One plain device copy of `nbytes` (reads nbytes, writes nbytes): the
    reference dispatch against which the byte counters are scaled."""
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def hold_cycles(torch, stream, seconds: float) -> int:
    """Argument of torch.cuda._sleep that holds the stream for about
    `seconds` (calibrated once here); 0 if this torch has no _sleep."""
    if not hasattr(torch.cuda, "_sleep"):
        return 0
    probe = 1 << 20
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(probe)
    e1.record(stream)
    torch.cuda.synchronize()
    per_cycle = max(e0.elapsed_time(e1) / 1e3, 1e-6) / probe
    return int(min(seconds / per_cycle, 1 << 34))


def hbm_copy_reference(torch, dev, nbytes: int = 1 << 30) -> dict:
    """The rate of a plain device copy (torch's copy of `nbytes`, best of
    three): what this part sustains for a simple streaming read + write, as
    context for the HBM roofline fractions (which use the 8 TB/s peak)."""
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(4):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del src, dst
    gbs = 2 * nbytes / best / 1e9
    return {"copy_bytes": nbytes, "copy_gbs": gbs, "copy_frac_of_peak": gbs / PEAK_HBM_GBS}


def dense_build_flops_per_token_head(d: int, c: int = CHUNK) -> float:
    """Algorithmic flops of the chunked dense build per token and head:
    the chunk's UT work 6*c*d (K K^T, U = A K, W = A V, each 2*c*d per token)
    plus the chain update 8*d^2 (U That, K^T N, U S, K^T M, each 2*d^2 per
    token)."""
    return 6.0 * c * d + 8.0 * d * d


def kda_build_flops_per_token_head(dk: int, dv: int) -> float:
    """Algorithmic flops of the token-by-token KDA build per token and head:
    for each element of S (dk x dv) and That (dk x dk), the gate's multiply
    (1), the column sum X^T k (2) and the rank-one update (2)."""
    return 5.0 * dk * (dk + dv)


def build_bytes(n_tok, layers, heads, dk, dv, n_seg, qkv_bytes=2):
    """Algorithmic bytes of one build: k and v once, alpha and beta once, the
    pairs out (That, S0, lambda)."""
    inp = n_tok * layers * heads * ((dk + dv) * qkv_bytes + 8)
    out = n_seg * layers * heads * (dk * dk + dk * dv + 1) * 4
    return inp + out


def compose_bytes(steps, layers, heads, dk, dv, n_req=1):
    """One compose: That_p and S0_p read per step, the state read and written once."""
    return steps * layers * heads * (dk * dk + dk * dv + 1) * 4 + 2 * n_req * layers * heads * dk * dv * 4


def naive_bytes(steps, layers, heads, dk, dv, n_req=1):
    return steps * layers * heads * dk * dv * 4 + n_req * layers * heads * dk * dv * 4


def cpu_baseline(w, seconds: float, threads: int):
    """The fp64 oracle (specialised path) on a bounded sample of the same
    workload: whole (layer, head, segment) units of 4096 tokens, drawn with the
    same distributions, as many as fit the time budget.  Returns prompt
    tokens/s extrapolated to all layers and heads."""
    import oracle
    import synth
    lib = oracle.load()
    L = w.seg_lens[0]
    # one (layer, segment) block: all heads; keep `threads` heads of it
    units_done = 0
    t0 = time.perf_counter()
    rounds = 0
    while True:
        x = synth.segment_inputs(w, layer=rounds % w.layers, seg_id=rounds % w.n_seg, L=L)
        h = min(threads, w.heads)
        k = x["k"][None, :, :h]
        v = x["v"][None, :, :h]
        a = x["alpha"][None, :, :h]
        b = x["beta"][None, :, :h]
        oracle.build(w.form, k, v, a, b, [0, L], threads=threads, lib=lib)
        units_done += h
        rounds += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    token_units_per_s = units_done * L / dt          # token x (layer, head) per second
    tokens_per_s = token_units_per_s / (w.layers * w.heads)
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{units_done} (layer, head, segment) units of {L} tokens on the fp64 "
                       f"oracle's specialised path in {dt:.1f} s; prompt tokens/s extrapolated "
                       f"to {w.layers} layers x {w.heads} heads (build only)")}


def bench_scalar_diag(w, args):
    """Scalar-decay or diagonal-gate workload: build every pair, compose the
    segments in order, naive add; one JSON line with HBM rooflines."""
    import torch
    import hybrid_caching_amd as pic
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pic.load()
    pic.pic_staging_reserve()  # asynchronous copies of large plan tables
    B, H, dk, dv, N, n_seg = w.layers, w.heads, w.dk, w.dv, w.n_tokens, w.n_seg
    offsets = w.offsets()
    qdt = torch.bfloat16 if w.qkv_bf16 else torch.float32
    ashape = (B, N, H, dk) if w.form == synth.DIAG else (B, N, H)
    k = torch.empty((B, N, H, dk), dtype=qdt, device=dev)
    v = torch.empty((B, N, H, dv), dtype=qdt, device=dev)
    alpha = torch.empty(ashape, dtype=torch.float32, device=dev)
    for layer in range(B):
        x = synth.torch_layer_inputs(w, layer, dev)
        k[layer].copy_(x["k"])
        v[layer].copy_(x["v"])
        alpha[layer].copy_(x["alpha"])
    lam_shape = (n_seg, B, H, dk) if w.form == synth.DIAG else (n_seg, B, H)
    pairs = {"log_scale": torch.empty(lam_shape, dtype=torch.float32, device=dev),
             "S0": torch.empty((n_seg, B, H, dk, dv), dtype=torch.float32, device=dev)}
    S_out = torch.empty((1, B, H, dk, dv), dtype=torch.float32, device=dev)
    S_naive = torch.empty_like(S_out)
    chain_off, chain_idx = [0, n_seg], list(range(n_seg))
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration)
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # Each kernel here runs for well under a millisecond, less than the host
    # needs to marshal and enqueue one call.  So each operation is timed as a
    # group of `reps` back-to-back launches that the host enqueues while the
    # stream is held by a spin kernel (torch.cuda._sleep) issued before the
    # group's first event: the events then see the launches run back to back
    # on the device, and the per-launch time is the group's time / reps.
    reps = args.reps
    # long enough for the host to enqueue the whole group (a few hundred
    # microseconds per call at worst)
    hold = hold_cycles(torch, stream, reps * 600e-6)

    def group(fn, e0, e1):
        if hold:
            torch.cuda._sleep(hold)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)

    def step(rec=None):
        e = [ev() for _ in range(6)]
        group(lambda: pic.pic_segment_build(w.form, k, v, alpha, None, offsets, out=pairs),
              e[0], e[1])
        group(lambda: pic.pic_compose(w.form, pairs["log_scale"], None, pairs["S0"], chain_off,
                                      chain_idx, None, out=S_out), e[2], e[3])
        group(lambda: pic.pic_naive_add(pairs["S0"], chain_off, chain_idx, None, out=S_naive),
              e[4], e[5])
        if rec is not None:
            rec.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    ms = [float(np.median([r[2 * i].elapsed_time(r[2 * i + 1]) for r in recs])) / reps
          for i in range(3)]
    kname = "build_diag_pipe_kernel" if w.form == synth.DIAG else "build_scalar_pipe_kernel"
    gate_bytes = 4 * (dk if w.form == synth.DIAG else 1)
    lam_out = 4 * (dk if w.form == synth.DIAG else 1)
    qb = 2 if w.qkv_bf16 else 4
    bb = N * B * H * ((dk + dv) * qb + gate_bytes) + n_seg * B * H * (dk * dv * 4 + lam_out)
    cb = n_seg * B * H * (dk * dv * 4 + lam_out) + B * H * dk * dv * 4
    nb = n_seg * B * H * dk * dv * 4 + B * H * dk * dv * 4
    flops = 2.0 * N * B * H * dk * dv
    gbs = lambda nbytes, t: nbytes / (t / 1e3) / 1e9
    out = {"metric": f"{synth.FORM_NAMES[w.form]} segment build tokens/s; % HBM roofline",
           "value": N / (ms[0] / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": float(sum(ms)), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32 state, bf16 k/v",
           "data": "synthetic",
           "config": {"workload": w.name, "form": synth.FORM_NAMES[w.form], "layers": B,
                      "heads": H, "dk": dk, "dv": dv, "segments": n_seg,
                      "segment_tokens": int(w.seg_lens[0]), "prompt_tokens": N,
                      "passes_per_step": reps},
           "ms": {"build": ms[0], "compose": ms[1], "naive_add": ms[2]},
           "roofline": {"kernel": kname, "bound": "hbm",
                        "achieved": gbs(bb, ms[0]), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs(bb, ms[0]) / PEAK_HBM_GBS,
                        "traffic": measured_traffic(kname, w.name),
                        "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": bb,
                        "tflops": flops / (ms[0] / 1e3) / 1e12},
           "roofline_compose": {"bound": "hbm", "achieved": gbs(cb, ms[1]),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": gbs(cb, ms[1]) / PEAK_HBM_GBS},
           "roofline_naive_add": {"bound": "hbm", "achieved": gbs(nb, ms[2]),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": gbs(nb, ms[2]) / PEAK_HBM_GBS},
           "hbm_reference": hbm_copy_reference(torch, dev)}
    print(json.dumps(out), flush=True)
    return 0


def bench_kda(w, args):
    """Delta rule with per-channel gates (KDA form): build every pair in one
    call, compose the segments in prompt order, naive add; one JSON line.
    At fp16 operand precision the build runs in chunks of 32 tokens on the
    matrix cores (roofline against the fp16 MFMA peak); at fp32 token by token
    on the vector units (fp32 VALU roofline).  The build at the other
    precision is timed as a secondary figure, outside `value`."""
    import torch
    import hybrid_caching_amd as pic
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pic.load()
    pic.pic_staging_reserve()  # asynchronous copies of large plan tables
    B, H, dk, dv, N, n_seg = w.layers, w.heads, w.dk, w.dv, w.n_tokens, w.n_seg
    offsets = w.offsets()
    qdt = torch.bfloat16 if w.qkv_bf16 else torch.float32
    prec = args.prec if (w.qkv_bf16 and dk == 128 and dv == 128) else 0
    k = torch.empty((B, N, H, dk), dtype=qdt, device=dev)
    v = torch.empty((B, N, H, dv), dtype=qdt, device=dev)
    alpha = torch.empty((B, N, H, dk), dtype=torch.float32, device=dev)
    beta = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    for layer in range(B):
        x = synth.torch_layer_inputs(w, layer, dev)
        k[layer].copy_(x["k"])
        v[layer].copy_(x["v"])
        alpha[layer].copy_(x["alpha"])
        beta[layer].copy_(x["beta"])
        del x
    pairs = {"log_scale": torch.empty((n_seg, B, H), dtype=torch.float32, device=dev),
             "T_hat": torch.empty((n_seg, B, H, dk, dk), dtype=torch.float32, device=dev),
             "S0": torch.empty((n_seg, B, H, dk, dv), dtype=torch.float32, device=dev)}
    S_out = torch.empty((1, B, H, dk, dv), dtype=torch.float32, device=dev)
    S_naive = torch.empty_like(S_out)
    chain_off, chain_idx = [0, n_seg], list(range(n_seg))
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration)
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(record=None):
        e = [ev() for _ in range(4)]
        e[0].record(stream)
        pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, out=pairs, precision=prec)
        e[1].record(stream)
        pic.pic_compose(w.form, pairs["log_scale"], pairs["T_hat"], pairs["S0"], chain_off,
                        chain_idx, None, out=S_out)
        e[2].record(stream)
        pic.pic_naive_add(pairs["S0"], chain_off, chain_idx, None, out=S_naive)
        e[3].record(stream)
        if record is not None:
            record.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    t_build, t_comp, t_naive = [float(np.mean([r[i].elapsed_time(r[i + 1]) for r in recs])) / 1e3
                                for i in range(3)]
    if prec:
        pic.pic_nonfinite_check(dev)  # the timed builds stayed inside fp16's range
    qb = 2 if w.qkv_bf16 else 4
    bb = N * B * H * ((dk + dv) * qb + 4 * dk + 4) + n_seg * B * H * (dk * dk + dk * dv + 1) * 4
    cb = compose_bytes(n_seg, B, H, dk, dv)
    nb = naive_bytes(n_seg, B, H, dk, dv)

    def build_roofline(p, t):
        if p:
            # the chunked KDA build works in chunks of 32 tokens
            flops = dense_build_flops_per_token_head(dk, 32) * N * B * H
            tf = flops / t / 1e12
            return {"kernel": "build_kda_chunk_kernel", "bound": "mfma", "achieved": tf,
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                    "traffic": measured_traffic("build_kda_chunk_kernel", w.name),
                    "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": bb,
                    "algorithmic_flops": flops}
        flops = kda_build_flops_per_token_head(dk, dv) * N * B * H
        tf = flops / t / 1e12
        return {"kernel": "build_kda_kernel", "bound": "alu", "achieved": tf,
                "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / PEAK_FP32_VALU_TFLOPS,
                "traffic": measured_traffic("build_kda_kernel", w.name),
                "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": bb,
                "algorithmic_flops": flops}

    out = {
        "metric": "KDA segment build tokens/s + state composes/s (H=32, d=128); "
                  "% of the build's roofline",
        "value": N / t_step, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_step * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("f16 matrix-core operands, f32 accumulation and state, bf16 k/v" if prec else
                  "f32 state and arithmetic, bf16 k/v" if w.qkv_bf16 else "f32"),
        "data": "synthetic",
        "config": {"workload": w.name, "form": "kda", "layers": B, "heads": H, "dk": dk,
                   "dv": dv, "segments": n_seg, "segment_tokens": int(w.seg_lens[0]),
                   "prompt_tokens": N, "build_precision": "fp16" if prec else "fp32"},
        "build_tokens_per_s": N / t_build,
        "composes_per_s": n_seg * B / t_comp,
        "ms": {"build": t_build * 1e3, "compose": t_comp * 1e3, "naive_add": t_naive * 1e3},
        "roofline": build_roofline(prec, t_build),
        "roofline_compose": {"kernel": "compose_dense_full_kernel", "bound": "hbm",
                             "achieved": cb / t_comp / 1e9, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": cb / t_comp / 1e9 / PEAK_HBM_GBS,
                             "algorithmic_bytes": cb},
        "roofline_naive_add": {"bound": "hbm", "achieved": nb / t_naive / 1e9,
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": nb / t_naive / 1e9 / PEAK_HBM_GBS},
    }
    if prec and not args.no_fp32_build:
        # the token-by-token fp32 build of the same inputs, for reference
        pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, out=pairs, precision=0)
        torch.cuda.synchronize()
        ts = []
        for _ in range(2):
            e0, e1 = ev(), ev()
            e0.record(stream)
            pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, out=pairs, precision=0)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        t32 = float(np.mean(ts))
        out["build_other_precision"] = {"precision": "fp32 (token by token)", "ms": t32 * 1e3,
                                        "tokens_per_s": N / t32,
                                        "roofline": build_roofline(0, t32)}
    if not args.no_cpu_baseline:
        try:
            threads = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            threads = min(16, os.cpu_count() or 1)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, threads)
    print(json.dumps(out), flush=True)
    return 0


def bench_split(w, args):
    """Few-unit launch (one long segment per layer): the build whole and cut
    into pieces that are built and merged (pic_segment_build split=n with
    n = suggest_split); one JSON line with both times, the split build's
    roofline and the two results' relative difference."""
    import torch
    import hybrid_caching_amd as pic
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pic.load()
    pic.pic_staging_reserve()
    B, H, dk, dv, N, n_seg = w.layers, w.heads, w.dk, w.dv, w.n_tokens, w.n_seg
    offsets = w.offsets()
    dense = w.form == synth.DENSE
    prec = args.prec if dense else 0
    x = synth.torch_layer_inputs(w, 0, dev)
    k, v, alpha = x["k"][None].contiguous(), x["v"][None].contiguous(), x["alpha"][None].contiguous()
    beta = x["beta"][None].contiguous() if x.get("beta") is not None else None
    n_split = pic.suggest_split(B, H, offsets)
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    outs = {}

    def timed(split):
        out = None
        for _ in range(args.warmup + 1):
            out = pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, precision=prec,
                                        split=split, out=out)
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.steps):
            e0, e1 = ev(), ev()
            e0.record(stream)
            pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, precision=prec,
                                  split=split, out=out)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        outs[split] = out
        return float(np.median(ts))

    t_whole = timed(1)
    t_split = timed(n_split)
    rel = float(torch.linalg.norm(outs[n_split]["S0"] - outs[1]["S0"]) /
                torch.linalg.norm(outs[1]["S0"]))
    if dense:
        flops = dense_build_flops_per_token_head(dk) * N * B * H
        roof = {"kernel": "build_dense_h16_kernel" if prec else "build_dense_ws_kernel",
                "bound": "mfma", "achieved": flops / t_split / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": flops / t_split / 1e12 / PEAK_BF16_TFLOPS,
                "algorithmic_flops": flops}
    else:
        nb = build_bytes(N, B, H, dk, dv, n_seg) - n_seg * B * H * dk * dk * 4
        roof = {"kernel": "build_scalar_pipe_kernel", "bound": "hbm",
                "achieved": nb / t_split / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": nb / t_split / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": nb}
    out = {
        "metric": "segment build tokens/s, few-unit launch: whole vs split into pieces and "
                  "merged by composition",
        "value": N / t_split, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_split * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("f32 state, bf16 k/v, fp16 MFMA operands" if prec else
                  "f32 state, bf16 k/v, split-bf16 MFMA"),
        "data": "synthetic",
        "config": {"workload": w.name, "form": synth.FORM_NAMES[w.form], "layers": B,
                   "heads": H, "dk": dk, "dv": dv, "segments": n_seg, "prompt_tokens": N,
                   "units": n_seg * B * H, "pieces_per_segment": n_split},
        "ms": {"whole": t_whole * 1e3, "split": t_split * 1e3},
        "speedup": t_whole / t_split,
        "split_vs_whole_rel_diff_S0": rel,
        "roofline": roof,
    }
    print(json.dumps(out), flush=True)
    return 0


def _group_segments(lens, max_tokens):
    """Consecutive runs of segments holding at most max_tokens tokens each."""
    groups, cur, tot = [], [], 0
    for i, n in enumerate(lens):
        if cur and tot + n > max_tokens:
            groups.append(cur)
            cur, tot = [], 0
        cur.append(i)
        tot += n
    if cur:
        groups.append(cur)
    return groups


def bench_reuse(w, args):
    """Composition-heavy reuse: build a pool of cached segments (all layers)
    and the requests' fresh segments, then compose every request's chain of
    pool and fresh pairs in one call.  Times the fresh builds (inputs resident
    per group of segments) and the batched compose; one JSON line."""
    import torch
    import hybrid_caching_amd as pic
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pic.load()
    pic.pic_staging_reserve()  # asynchronous copies of large plan tables
    fw = synth.reuse_fresh_workload(w)
    off, idx = synth.reuse_chains(w)
    B, H, dk, dv = w.layers, w.heads, w.dk, w.dv
    n_pool, n_fresh = w.n_seg, fw.n_seg
    P = n_pool + n_fresh
    R = len(off) - 1
    pool = {"log_scale": torch.empty((P, B, H), dtype=torch.float32, device=dev),
            "T_hat": torch.empty((P, B, H, dk, dk), dtype=torch.float32, device=dev),
            "S0": torch.empty((P, B, H, dk, dv), dtype=torch.float32, device=dev)}
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def build_groups(wl, base, seed_base, record):
        lens = list(wl.seg_lens)
        for gi, grp in enumerate(_group_segments(lens, 32768)):
            gl = [lens[i] for i in grp]
            gw = synth.scaled(wl, seg_lens=gl, name=wl.name)
            Ng = sum(gl)
            k = torch.empty((B, Ng, H, dk), dtype=torch.bfloat16, device=dev)
            v = torch.empty((B, Ng, H, dv), dtype=torch.bfloat16, device=dev)
            alpha = torch.empty((B, Ng, H), dtype=torch.float32, device=dev)
            beta = torch.empty((B, Ng, H), dtype=torch.float32, device=dev)
            for layer in range(B):
                x = synth.torch_layer_inputs(gw, layer, dev, seed_offset=seed_base + 131 * gi)
                k[layer].copy_(x["k"])
                v[layer].copy_(x["v"])
                alpha[layer].copy_(x["alpha"])
                beta[layer].copy_(x["beta"])
                del x
            p0, p1 = base + grp[0], base + grp[-1] + 1
            out = {key: t[p0:p1] for key, t in pool.items()}
            goff = np.concatenate([[0], np.cumsum(gl)]).astype(np.int64)
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record(stream)
            pic.pic_segment_build(synth.DENSE, k, v, alpha, beta, goff, out=out,
                                  precision=args.prec)
            e1.record(stream)
            record.append((e0, e1, Ng))
            del k, v, alpha, beta

    pool_rec, fresh_rec = [], []
    t0 = time.perf_counter()
    build_groups(w, 0, 0, pool_rec)
    build_groups(fw, n_pool, 7, fresh_rec)
    torch.cuda.synchronize()
    prep_s = time.perf_counter() - t0
    fresh_ms = sum(a.elapsed_time(b) for a, b, _ in fresh_rec)
    fresh_tokens = sum(n for _, _, n in fresh_rec)

    S_out = torch.empty((R, B, H, dk, dv), dtype=torch.float32, device=dev)
    seam_w = int(w.extra.get("seam", 0))
    if seam_w:
        seam_off = synth.reuse_seam_offsets(off, seam_w)
        n_seam = int(seam_off[-1])
        si = synth.torch_seam_inputs(w, n_seam, dev)
        O = torch.empty((B, n_seam, H, dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration)

    def compose():
        if seam_w:
            pic.pic_compose_seams(synth.DENSE, pool["log_scale"], pool["T_hat"], pool["S0"], off,
                                  idx, seam_off, si["q"], si["k"], si["v"], si["alpha"],
                                  si["beta"], None, out=S_out, out_O=O)
        else:
            pic.pic_compose(synth.DENSE, pool["log_scale"], pool["T_hat"], pool["S0"], off, idx,
                            None, out=S_out)

    for _ in range(max(args.warmup, 1)):
        compose()
    torch.cuda.synchronize()
    recs = []
    for _ in range(args.steps):
        e0, e1 = ev(), ev()
        e0.record(stream)
        compose()
        e1.record(stream)
        recs.append((e0, e1))
    torch.cuda.synchronize()
    t_comp = float(np.mean([a.elapsed_time(b) for a, b in recs])) / 1e3
    steps_total = int(off[-1])
    composes = steps_total * B                     # pair applications per layer, all heads
    # every step reads its pair once; the states are written once (no S_in)
    cb = compose_bytes(steps_total, B, H, dk, dv, n_req=0) + R * B * H * dk * dv * 4
    kname, seam_info = "compose_dense_full_kernel", None
    if seam_w:
        # each seam token reads q, k, v (bf16), alpha, beta and writes its output
        # (fp32); its update u = S^T k, S <- a S + k c^T, o = S^T q is 7 dk dv flops
        tok_bytes = B * H * ((2 * dk + dv) * 2 + 8 + dv * 4)
        cb += n_seam * tok_bytes
        seam_flops = 7.0 * dk * dv * n_seam * B * H
        t_valu = seam_flops / (PEAK_FP32_VALU_TFLOPS * 1e12)
        kname = "compose_seam_kernel"
        seam_info = {"window": seam_w, "seam_tokens": n_seam, "seam_flops": seam_flops,
                     "valu_time_at_peak_ms": t_valu * 1e3,
                     "hbm_time_at_peak_ms": cb / (PEAK_HBM_GBS * 1e9) * 1e3,
                     "output_tokens_per_s": n_seam * B / t_comp}
    conv_info = None
    if seam_w:
        # convolution warm-up of width 4 (windows of 3 tokens) for every chain
        # entry, one call per stream (q, k, v), over the seam inputs as the raw
        # store; not part of `value`
        cw = 4
        n_e = steps_total
        heads_at = [int(min(seam_off[c], n_seam - (cw - 1))) for c in range(n_e)]
        hist = [int(min(cw - 1, h)) for h in heads_at]
        wts = {nm: torch.randn((H, d, cw), generator=torch.Generator(device=dev).manual_seed(5),
                               device=dev) / cw for nm, d in (("q", dk), ("k", dk), ("v", dv))}
        ys = {nm: torch.empty((B, n_e * (cw - 1), H, si[nm].shape[-1]), dtype=si[nm].dtype,
                              device=dev) for nm in ("q", "k", "v")}

        def warm():
            for nm in ("q", "k", "v"):
                pic.pic_conv_warmup(wts[nm], si[nm], heads_at, heads_at, hist, cw - 1,
                                    out=ys[nm])

        warm()
        torch.cuda.synchronize()
        cr = []
        for _ in range(3):
            e0, e1 = ev(), ev()
            e0.record(stream)
            warm()
            e1.record(stream)
            cr.append((e0, e1))
        torch.cuda.synchronize()
        t_cw = float(np.mean([a.elapsed_time(b) for a, b in cr])) / 1e3 / 3  # per launch
        # per launch (one stream; q, k, v have d = 128 here), bf16: each output
        # token written once, each entry's head and history tokens read once
        cwb = 3 * B * H * dk * n_e * (cw - 1) * 2
        # (width 4 with up to 13 outputs per entry runs the window-in-registers
        # kernel, other widths the general one)
        conv_kernel = "conv_warmup_w4_kernel" if cw == 4 else "conv_warmup_kernel"
        conv_info = {"kernel": conv_kernel, "width": cw, "entries": n_e,
                     "tokens": n_e * (cw - 1), "ms_per_launch": t_cw * 1e3,
                     "launches": "3 (q, k, v)", "bound": "hbm",
                     "achieved": cwb / t_cw / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": cwb / t_cw / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": cwb,
                     "traffic": measured_traffic(conv_kernel, w.name)}
    gbs = cb / t_comp / 1e9
    out = {"metric": "state composes/s (dense delta, H=32, d=128), composition-heavy reuse"
                     + (" with seam windows" if seam_w else "") + "; % HBM roofline",
           "value": composes / t_comp, "unit": "composes/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": t_comp * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32 state, split-bf16 MFMA",
           "data": "synthetic",
           "config": {"workload": w.name, "form": "dense_gdn", "layers": B, "heads": H, "dk": dk,
                      "dv": dv, "build_precision": args.precision, "pool_segments": n_pool, "requests": R,
                      "chain_steps": steps_total // R, "fresh_segments": n_fresh,
                      "fresh_segment_tokens": int(fw.seg_lens[0])},
           "roofline": {"kernel": kname, "bound": "hbm", "achieved": gbs,
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                        "traffic": measured_traffic(kname, w.name),
                        "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": cb},
           "fresh_build": {"tokens_per_s": fresh_tokens / (fresh_ms / 1e3), "ms": fresh_ms,
                           "segments": n_fresh, "layers": B},
           "seam": seam_info,
           "conv_warmup": conv_info,
           "pool_and_input_preparation_s": prep_s,
           "hbm_reference": hbm_copy_reference(torch, dev)}
    print(json.dumps(out), flush=True)
    return 0


def run_leg(name: str, args, keep):
    """One workload's bench line from a child process (this file, --workload
    name), reduced to the keys in `keep`; an error entry if it fails."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--no-cpu-baseline",
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--precision",
           args.precision]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if res.returncode != 0:
        return {"error": f"exit {res.returncode}", "stderr": res.stderr[-400:]}
    line = [x for x in res.stdout.splitlines() if x.startswith("{")][-1]
    d = json.loads(line)
    return {key: d[key] for key in keep if d.get(key) is not None}


def prefill_flops_per_token_head(dk: int, dv: int, track_T: bool, sub: int = 32) -> float:
    """Matrix-core work of the prefill with outputs per token and head, at the
    kernel's sub-chunks of `sub` tokens: K K^T (2 sub dk), Y = K S (2 dk dv),
    the W seed and A Y (2 sub dv each), S += K^T P (2 dk dv), the outputs Q S
    (2 dk dv), K Q^T (2 sub dk) and (K Q^T)^T P (2 sub dv); tracking That adds
    K That, A Y and That += K^T N (2 dk^2 + 2 sub dk + 2 dk^2)."""
    f = 2.0 * sub * dk + 2 * dk * dv + 4.0 * sub * dv + 2 * dk * dv + 2 * dk * dv \
        + 2.0 * sub * dk + 2.0 * sub * dv
    if track_T:
        f += 4.0 * dk * dk + 2.0 * sub * dk
    return f


def prefill_leg(w, k, v, alpha, beta, pairs, args):
    """The prefill with per-token outputs over the whole workload (one call for
    all segments, layers and heads), without and with That: times, rates and
    the measured overhead of building the pair in the prefill."""
    import torch
    import hybrid_caching_amd as pic
    import synth
    dev = k.device
    B, N, H = k.shape[0], k.shape[1], k.shape[2]
    dk, dv = k.shape[3], v.shape[3]
    q = torch.empty_like(k)
    for layer in range(B):
        q[layer].copy_(synth.torch_layer_queries(w, layer, dev))
    O = torch.empty((B, N, H, dv), dtype=torch.bfloat16, device=dev)
    offsets = w.offsets()
    stream = torch.cuda.current_stream(dev)
    res = {}
    for track in (False, True):
        out = {"log_scale": pairs["log_scale"], "S0": pairs["S0"], "O": O}
        if track:
            out["T_hat"] = pairs["T_hat"]
        run = lambda: pic.pic_segment_prefill(q, k, v, alpha, beta, offsets, track_T=track,
                                              out=out)
        for _ in range(max(1, args.warmup)):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, args.steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        res[track] = float(np.mean(ts))
    del q, O
    th = N * B * H
    nbytes = th * ((2 * dk + dv) * 2 + 8 + dv * 2)  # q, k, v, alpha, beta in; O out (bf16)
    legs = {}
    for track, name in ((False, "prefill"), (True, "prefill_with_pair")):
        t = res[track]
        pb = w.n_seg * B * H * ((dk * dk if track else 0) + dk * dv + 1) * 4
        fl = prefill_flops_per_token_head(dk, dv, track) * th
        bb = nbytes + pb
        t_hbm, t_mfma = bb / (PEAK_HBM_GBS * 1e9), fl / (PEAK_BF16_TFLOPS * 1e12)
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        # the two launches are two instantiations of the kernel; the counter
        # summary keys them by workload name (with "_pair" for That tracked)
        traffic = measured_traffic("dense_fp16_kernel", w.name + ("_pair" if track else ""))
        legs[name] = {"kernel": "dense_fp16_kernel", "ms": t * 1e3, "tokens_per_s": N / t,
                      "output_token_heads_per_s": th / t,
                      "roofline": {"bound": bound,
                                   "achieved": bb / t / 1e9 if bound == "hbm" else fl / t / 1e12,
                                   "peak": PEAK_HBM_GBS if bound == "hbm" else PEAK_BF16_TFLOPS,
                                   "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                                   "frac": (t_hbm if bound == "hbm" else t_mfma) / t,
                                   "algorithmic_bytes": bb, "algorithmic_flops": fl,
                                   "mfma_frac": t_mfma / t, "traffic": traffic,
                                   "traffic_unit": "HBM bytes per launch"}}
    legs["pair_overhead_in_prefill"] = res[True] / res[False] - 1.0
    return legs


def phase_timing(w, args) -> int:
    """Per-role clocks of the dense fp16 build (diagnostic): runs one build of
    `w` (by default 2 of its layers) through ``libpic_timing.so``, whose dense
    fp16 kernel records, per wave, each pipeline phase's length and the wait at
    its closing barrier, and prints per role the mean clocks per 64-token cycle:
    phase A / phase B length, busy time (length - wait) and the cycle total."""
    import ctypes
    import torch
    import synth
    from hybrid_caching_amd import _build, _lib
    if not os.path.exists(_build.TIMING_LIB_PATH):
        raise SystemExit(f"{_build.TIMING_LIB_PATH} is missing: run the build first")
    lib = _lib.load(_build.TIMING_LIB_PATH)
    lib.pic_phase_timing_set.restype = ctypes.c_int
    lib.pic_phase_timing_set.argtypes = [ctypes.c_void_p, ctypes.c_int]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = args.layers or 2
    w = synth.scaled(w, layers=layers, name=w.name)
    B, H, dk, dv, N, n_seg = w.layers, w.heads, w.dk, w.dv, w.n_tokens, w.n_seg
    k = torch.empty((B, N, H, dk), dtype=torch.bfloat16, device=dev)
    v = torch.empty((B, N, H, dv), dtype=torch.bfloat16, device=dev)
    alpha = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    beta = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    for layer in range(B):
        x = synth.torch_layer_inputs(w, layer, dev)
        k[layer].copy_(x["k"])
        v[layer].copy_(x["v"])
        alpha[layer].copy_(x["alpha"])
        beta[layer].copy_(x["beta"])
        del x
    lam = torch.empty((n_seg, B, H), dtype=torch.float32, device=dev)
    T = torch.empty((n_seg, B, H, dk, dk), dtype=torch.float32, device=dev)
    S = torch.empty((n_seg, B, H, dk, dv), dtype=torch.float32, device=dev)
    blocks = n_seg * B * H
    out = torch.zeros((blocks, 8, 8), dtype=torch.int64, device=dev)
    off = np.ascontiguousarray(np.asarray(w.offsets(), dtype=np.int64))
    ws = torch.empty(max(int(lib.pic_segment_build_workspace(2, B, H, dk, dv, N, n_seg)), 256),
                     dtype=torch.uint8, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if lib.pic_phase_timing_set(P(out), blocks) != 0:
        raise SystemExit("pic_phase_timing_set failed")
    for _ in range(2):  # the second run is the one read
        rc = lib.pic_segment_build(2, 1, 1, B, H, dk, dv, N, None, P(k), P(v), P(alpha), P(beta),
                                   off.ctypes.data_as(ctypes.c_void_p), n_seg, P(lam), P(T), P(S),
                                   P(ws), ws.numel(), stream)
        if rc != 0:
            raise SystemExit(f"build failed: {lib.pic_last_error().decode()}")
        torch.cuda.synchronize()
    r = out.cpu().numpy().astype(np.float64)  # [block][wave][field]
    cyc = np.maximum(r[:, :, 5], 1)
    roles = {"consumer": [0, 1, 2, 3], "solver": [4], "K staging": [5, 6], "V staging": [7]}
    rows = {}
    for name, waves in roles.items():
        x = r[:, waves]
        c = cyc[:, waves]
        lenA, waitA = (x[..., 0] / c).mean(), (x[..., 1] / c).mean()
        lenB, waitB = (x[..., 2] / c).mean(), (x[..., 3] / c).mean()
        rows[name] = {"phase_A": round(lenA), "busy_A": round(lenA - waitA),
                      "phase_B": round(lenB), "busy_B": round(lenB - waitB),
                      "cycle": round((x[..., 4] / c).mean())}
    print(json.dumps({"phase_timing": "build_dense_h16_kernel", "workload": w.name,
                      "layers": layers, "clocks_per_64_token_cycle": rows}))
    for name, row in rows.items():
        print(f"{name:10s} " + "  ".join(f"{k} {v:6d}" for k, v in row.items()), file=sys.stderr)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="dense_30L_32x4096")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--precision", choices=["fp32", "fp16"], default="fp16",
                    help="operand precision of the dense build's matrix-core products: fp16 "
                         "(single fp16 operands, the default; relative error ~2e-3 against the "
                         "fp64 oracle) or fp32 (split bf16, ~2e-5); state and accumulation are "
                         "fp32 in both")
    ap.add_argument("--no-fp32-build", action="store_true",
                    help="skip the secondary timing of the dense build at fp32 operand precision")
    ap.add_argument("--reps", type=int, default=20,
                    help="scalar/diagonal workloads: passes of each operation per timed step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run one plain device copy of BYTES (read BYTES, write BYTES) before "
                         "timing, as a reference for hardware byte counters")
    ap.add_argument("--no-legs", action="store_true",
                    help="default workload: skip the extra legs (prefill with outputs, scalar, "
                         "diagonal, reuse)")
    ap.add_argument("--no-child-legs", action="store_true",
                    help="default workload: keep the prefill leg (this process) but skip the "
                         "scalar, diagonal and reuse legs (child processes), e.g. under a "
                         "profiler")
    ap.add_argument("--phase-timing", action="store_true",
                    help="diagnostic: per-role clocks per pipeline cycle of the dense fp16 build "
                         "(loads libpic_timing.so; 2 layers unless --layers)")
    ap.add_argument("--source-digest", action="store_true",
                    help="print the source digest of each timed kernel and exit")
    args = ap.parse_args(argv)
    args.prec = 1 if args.precision == "fp16" else 0
    if args.source_digest:
        for kname in KERNEL_SOURCES:
            print(kname, source_digest(kname))
        return 0

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import hybrid_caching_amd as pic
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.phase_timing:
        return phase_timing(w, args)
    if args.layers:
        w = synth.scaled(w, layers=args.layers, name=w.name)
    if w.extra.get("split_demo"):
        return bench_split(w, args)
    if w.form == synth.KDA:
        return bench_kda(w, args)
    if w.form != synth.DENSE:
        return bench_scalar_diag(w, args)
    if w.extra.get("pool_size"):
        return bench_reuse(w, args)
    child_legs = {}
    if not args.no_legs and not args.no_child_legs and w.name == "dense_30L_32x4096":
        # the other workloads, each in a process of its own, run before this
        # process touches the device (their timings then see no other context)
        keep = ("value", "unit", "ms", "roofline", "roofline_compose", "roofline_naive_add",
                "fresh_build", "build_other_precision", "speedup", "config")
        for name in ("scalar_8x2048", "diag_16x4096", "reuse_256x30", "kda_30L_32x4096",
                     "few_dense_1x65536"):
            child_legs[name] = run_leg(name, args, keep)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pic.load()
    pic.pic_staging_reserve()  # asynchronous copies of large plan tables
    B, H, dk, dv, N, n_seg = w.layers, w.heads, w.dk, w.dv, w.n_tokens, w.n_seg
    offsets = w.offsets()

    # ---- inputs resident in HBM
    qdt = torch.bfloat16 if w.qkv_bf16 else torch.float32
    k = torch.empty((B, N, H, dk), dtype=qdt, device=dev)
    v = torch.empty((B, N, H, dv), dtype=qdt, device=dev)
    alpha = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    beta = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    for layer in range(B):
        x = synth.torch_layer_inputs(w, layer, dev)
        k[layer].copy_(x["k"])
        v[layer].copy_(x["v"])
        alpha[layer].copy_(x["alpha"])
        beta[layer].copy_(x["beta"])
        del x
    pairs = {"log_scale": torch.empty((n_seg, B, H), dtype=torch.float32, device=dev),
             "T_hat": torch.empty((n_seg, B, H, dk, dk), dtype=torch.float32, device=dev),
             "S0": torch.empty((n_seg, B, H, dk, dv), dtype=torch.float32, device=dev)}
    S_out = torch.empty((1, B, H, dk, dv), dtype=torch.float32, device=dev)
    S_naive = torch.empty_like(S_out)
    chain_off, chain_idx = [0, n_seg], list(range(n_seg))
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration)

    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(record=None):
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record(stream)
        pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, out=pairs,
                              precision=args.prec)
        e1.record(stream)
        pic.pic_compose(w.form, pairs["log_scale"], pairs["T_hat"], pairs["S0"], chain_off,
                        chain_idx, None, out=S_out)
        e2.record(stream)
        pic.pic_naive_add(pairs["S0"], chain_off, chain_idx, None, out=S_naive)
        e3.record(stream)
        if record is not None:
            record.append((e0, e1, e2, e3))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_build = np.mean([a.elapsed_time(b) for a, b, _, _ in recs]) / 1e3
    t_comp = np.mean([b.elapsed_time(c) for _, b, c, _ in recs]) / 1e3
    t_naive = np.mean([c.elapsed_time(d) for _, _, c, d in recs]) / 1e3
    t_step_ev = np.mean([a.elapsed_time(d) for a, _, _, d in recs]) / 1e3
    t_step = wall / args.steps

    flops = dense_build_flops_per_token_head(dk) * N * B * H
    achieved_tf = flops / t_build / 1e12
    # the same build at the other operand precision, for reference (not in `value`)
    other = None
    if not args.no_fp32_build and args.prec == 1:
        pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, out=pairs, precision=0)
        torch.cuda.synchronize()
        evs = []
        for _ in range(3):
            e0, e1 = ev(), ev()
            e0.record(stream)
            pic.pic_segment_build(w.form, k, v, alpha, beta, offsets, out=pairs, precision=0)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t_other = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evs])) / 1e3
        other = {"precision": "fp32 (split bf16)", "kernel": "build_dense_ws_kernel",
                 "ms": t_other * 1e3, "build_tokens_per_s": N / t_other,
                 "achieved_tflops": flops / t_other / 1e12,
                 "frac_of_bf16_peak": flops / t_other / 1e12 / PEAK_BF16_TFLOPS}
    # re-rotation of every built pair to a new offset (rotary embeddings on the
    # keys, rot_dim = d_k, half pairing), out of place; not part of `value`
    rr_shift = [int(x) for x in np.cumsum([0] + list(w.seg_lens[:-1]))]
    moved = {"log_scale": torch.empty_like(pairs["log_scale"]),
             "T_hat": torch.empty_like(pairs["T_hat"]), "S0": torch.empty_like(pairs["S0"])}
    rr = lambda: pic.pic_rerotate(w.form, pairs["log_scale"], pairs["T_hat"], pairs["S0"],
                                  list(range(n_seg)), rr_shift, dk, 10000.0, pic.ROPE_HALF,
                                  out=moved)
    rr()
    torch.cuda.synchronize()
    evs = []
    for _ in range(3):
        e0, e1 = ev(), ev()
        e0.record(stream)
        rr()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    t_rr = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evs])) / 1e3
    rrb = 2 * n_seg * B * H * (dk * dk + dk * dv + 1) * 4
    composes = n_seg * B  # pairs applied to a running state, per layer (all heads)
    build_kernel = "build_dense_h16_kernel" if args.prec else "build_dense_ws_kernel"
    cb = compose_bytes(n_seg, B, H, dk, dv)
    nb = naive_bytes(n_seg, B, H, dk, dv)
    out = {
        "metric": METRIC,
        "value": N / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32 state, bf16 k/v, fp16 MFMA operands" if args.prec else
                  "f32 state, bf16 k/v, split-bf16 MFMA"),
        "data": "synthetic",
        "config": {"workload": w.name, "form": "dense_gdn", "layers": B, "heads": H, "dk": dk,
                   "dv": dv, "build_precision": args.precision, "segments": n_seg, "segment_tokens": int(w.seg_lens[0]),
                   "prompt_tokens": N, "chunk": CHUNK},
        "build_tokens_per_s": N / t_build,
        "composes_per_s": composes / t_comp,
        "ms": {"build": t_build * 1e3, "compose": t_comp * 1e3, "naive_add": t_naive * 1e3,
               "step_events": t_step_ev * 1e3},
        "roofline": {"kernel": build_kernel, "bound": "mfma", "achieved": achieved_tf,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved_tf / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(build_kernel, w.name),
                     "traffic_unit": "HBM bytes per launch",
                     "algorithmic_bytes": build_bytes(N, B, H, dk, dv, n_seg)},
        "roofline_compose": {"kernel": "compose_dense_full_kernel", "bound": "hbm",
                             "achieved": cb / t_comp / 1e9, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": cb / t_comp / 1e9 / PEAK_HBM_GBS,
                             "traffic": measured_traffic("compose_dense_full_kernel", w.name),
                             "algorithmic_bytes": cb},
        "roofline_naive_add": {"bound": "hbm", "achieved": nb / t_naive / 1e9,
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": nb / t_naive / 1e9 / PEAK_HBM_GBS},
        "build_hbm_gbs": build_bytes(N, B, H, dk, dv, n_seg) / t_build / 1e9,
        "rerotate": {"kernel": "rerotate_kernel", "pairs": n_seg * B * H, "ms": t_rr * 1e3,
                     "bound": "hbm", "achieved": rrb / t_rr / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": rrb / t_rr / 1e9 / PEAK_HBM_GBS,
                     "algorithmic_bytes": rrb,
                     "traffic": measured_traffic("rerotate_kernel", w.name)},
    }
    if other is not None:
        out["build_other_precision"] = other
    out["hbm_reference"] = hbm_copy_reference(torch, dev)
    if not args.no_legs and w.name == "dense_30L_32x4096":
        # the other parts of the path, measured in the same run (each with its
        # own roofline; not part of `value`)
        legs = prefill_leg(w, k, v, alpha, beta, pairs, args)
        legs["pair_overhead_vs_separate_build"] = t_build / (legs["prefill"]["ms"] / 1e3)
        legs.update(child_legs)
        out["legs"] = legs
    if not args.no_cpu_baseline:
        try:
            threads = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            threads = min(16, os.cpu_count() or 1)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, threads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
