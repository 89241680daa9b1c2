"""ctypes binding of ``libpic.so`` (the C ABI declared in ``include/pic.h``).

Argument marshalling only: every step of the segment transform runs in the
HIP kernels of the library.  torch supplies device memory and the stream.
There is no fallback: if the library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpic.so")

FORM_SCALAR, FORM_DIAG, FORM_DENSE, FORM_KDA = 0, 1, 2, 3
ROPE_INTERLEAVED, ROPE_HALF = 0, 1
_HAS_T_HAT = (FORM_DENSE, FORM_KDA)
DT_F32, DT_BF16 = 0, 1
PREC_FP32, PREC_FP16 = 0, 1

STATUS = {0: "PIC_OK", -1: "PIC_ERR_NULL", -2: "PIC_ERR_DIMS", -3: "PIC_ERR_OFFSETS",
          -4: "PIC_ERR_CHAIN", -5: "PIC_ERR_WORKSPACE", -6: "PIC_ERR_UNSUPPORTED",
          -7: "PIC_ERR_HIP", -8: "PIC_ERR_ALIGN", -9: "PIC_ERR_NONFINITE"}

_i, _i32, _i64, _sz, _p = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/pic.h
SIGNATURES = {
    "pic_abi_version": (_i, []),
    "pic_status_string": (ctypes.c_char_p, [_i]),
    "pic_last_error": (ctypes.c_char_p, []),
    "pic_segment_build_workspace": (_sz, [_i, _i, _i, _i, _i, _i64, _i32]),
    "pic_validate_build": (_i, [_i, _i, _i, _i, _i, _i, _i, _i64, _p, _p, _p, _p, _p, _p, _i32, _p,
                                _p, _p, _p, _sz]),
    "pic_segment_build": (_i, [_i, _i, _i, _i, _i, _i, _i, _i64, _p, _p, _p, _p, _p, _p, _i32, _p,
                               _p, _p, _p, _sz, _p]),
    "pic_segment_build_split_workspace": (_sz, [_i, _i, _i, _i, _i, _i64, _i32, _i32]),
    "pic_split_plan": (_i, [_i32, _p, _i64, _i32, _p, _i64, _p, _p]),
    "pic_segment_build_split": (_i, [_i, _i, _i, _i, _i, _i, _i, _i64, _p, _p, _p, _p, _p, _p,
                                     _i32, _i32, _p, _p, _p, _p, _sz, _p]),
    "pic_validate_prefill": (_i, [_i, _i, _i, _i, _i64, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _p,
                                  _p, _p, _sz]),
    "pic_segment_prefill": (_i, [_i, _i, _i, _i, _i64, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _p,
                                 _p, _p, _sz, _p]),
    "pic_compose_workspace": (_sz, [_i32, _i64]),
    "pic_validate_compose": (_i, [_i, _i, _i, _i, _i, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _p,
                                  _p, _p, _sz]),
    "pic_compose": (_i, [_i, _i, _i, _i, _i, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _p, _p, _p,
                         _sz, _p]),
    "pic_validate_naive_add": (_i, [_i, _i, _i, _i, _i64, _p, _i32, _p, _p, _p, _p, _p, _sz]),
    "pic_naive_add": (_i, [_i, _i, _i, _i, _i64, _p, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "pic_compose_seams_workspace": (_sz, [_i32, _i64]),
    "pic_validate_compose_seams": (_i, [_i, _i, _i, _i, _i, _i, _i64, _p, _p, _p, _i32, _p, _p, _p,
                                        _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz]),
    "pic_compose_seams": (_i, [_i, _i, _i, _i, _i, _i, _i64, _p, _p, _p, _i32, _p, _p, _p, _i64,
                               _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "pic_materialize_T": (_i, [_i, _i64, _i, _p, _p, _p, _p]),
    "pic_conv_warmup_workspace": (_sz, [_i32]),
    "pic_validate_conv_warmup": (_i, [_i, _i, _i, _i, _i, _i64, _p, _p, _i32, _i32, _p, _p, _p, _p,
                                      _p, _sz]),
    "pic_conv_warmup": (_i, [_i, _i, _i, _i, _i, _i64, _p, _p, _i32, _i32, _p, _p, _p, _p, _p, _sz,
                             _p]),
    "pic_rerotate_workspace": (_sz, [_i32]),
    "pic_validate_rerotate": (_i, [_i, _i, _i, _i, _i, _i64, _p, _p, _p, _i32, _p, _p, _i,
                                   ctypes.c_double, _i, _p, _p, _p, _p, _sz]),
    "pic_rerotate": (_i, [_i, _i, _i, _i, _i, _i64, _p, _p, _p, _i32, _p, _p, _i, ctypes.c_double,
                          _i, _p, _p, _p, _p, _sz, _p]),
    "pic_plan_dump": (_i, [_i, _i32, _p, _p, _i64, _p, _i64]),
    "pic_compose_noalloc": (_i, [_i, _i, _i, _i, _i, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _p,
                                 _p, _p]),
    "pic_staging_reserve": (_i, []),
    "pic_staging_release": (_i, []),
    "pic_staging_bytes": (_sz, []),
    "pic_nonfinite_check": (_i, [_p]),
}

PLAN_BUILD, PLAN_COMPOSE = 0, 1
PLAN_BUILD_COLS, PLAN_COMPOSE_COLS = 5, 3

_LIB = None


class PicError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(code, code)}: {detail}")
        self.code = code


def load(path: str = LIB_PATH):
    """Load libpic.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m hybrid_caching_amd._build`"
                          " (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _LIB = lib
    return lib


def _check(code: int, where: str):
    if code != 0:
        raise PicError(code, where, load().pic_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _host_i64(x):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _host_i32(x):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    if a.size == 0:
        a = np.zeros(1, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _need(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _workspace(nbytes: int, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def suggest_split(batch: int, heads: int, seg_offsets, units_wanted: int = 512,
                  min_piece_tokens: int = 1024) -> int:
    """Pieces per segment for pic_segment_build(split=...): 1 when the launch
    already has units_wanted (segment, layer, head) units, else enough pieces
    to reach it, none shorter than min_piece_tokens (of the longest segment)."""
    off = [int(x) for x in seg_offsets]
    n_seg = len(off) - 1
    units = n_seg * batch * heads
    if units >= units_wanted or n_seg == 0:
        return 1
    longest = max(off[i + 1] - off[i] for i in range(n_seg))
    want = -(-units_wanted // units)
    return max(1, min(want, longest // min_piece_tokens))


def pic_segment_build(form: int, k, v, alpha, beta, seg_offsets, q=None, *, out=None,
                      precision: int = PREC_FP32, check_finite: bool = False, split: int = 1):
    """Cached pairs of every (segment, layer, head).

    k: [B, N, H, dk], v: [B, N, H, dv] (both bf16 or both fp32), alpha: fp32
    [B, N, H] (diag, KDA: [B, N, H, dk]), beta: fp32 [B, N, H] or None (= 1;
    dense and KDA only), seg_offsets: host ints [n_seg+1].  precision:
    PREC_FP32 or PREC_FP16 (dense with bf16 k/v; KDA with bf16 k/v and
    dk = dv = 128).  Returns
    dict(log_scale, T_hat (dense and KDA only), S0) of fp32 device tensors
    laid out [n_seg, B, H, ...].  check_finite (PREC_FP16): wait for the
    stream and raise PicError when an fp16 operand overflowed (see
    pic_nonfinite_check).  split > 1: every segment is cut into up to `split`
    pieces of whole 64-token chunks whose pairs are built and merged in order
    (pic_segment_build_split; see suggest_split).
    """
    lib = load()
    B, N, H, dk = k.shape
    dv = v.shape[3]
    if k.dtype != v.dtype or k.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("k and v must both be bfloat16 or both float32")
    dt = DT_BF16 if k.dtype == torch.bfloat16 else DT_F32
    for t, n, d in ((k, "k", None), (v, "v", None), (alpha, "alpha", torch.float32),
                    (beta, "beta", torch.float32), (q, "q", None)):
        _need(t, n, d)
    offs, offs_p = _host_i64(seg_offsets)
    n_seg = len(offs) - 1
    dev = k.device
    if out is None:
        lam_shape = (n_seg, B, H, dk) if form == FORM_DIAG else (n_seg, B, H)
        out = {"log_scale": torch.empty(lam_shape, dtype=torch.float32, device=dev),
               "S0": torch.empty((n_seg, B, H, dk, dv), dtype=torch.float32, device=dev)}
        if form in _HAS_T_HAT:
            out["T_hat"] = torch.empty((n_seg, B, H, dk, dk), dtype=torch.float32, device=dev)
    if split > 1:
        ws_n = lib.pic_segment_build_split_workspace(form, B, H, dk, dv, N, n_seg, int(split))
        ws = _workspace(ws_n, dev)
        rc = lib.pic_segment_build_split(form, dt, precision, B, H, dk, dv, N, _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(alpha), _ptr(beta), offs_p, n_seg,
                                         int(split), _ptr(out["log_scale"]), _ptr(out.get("T_hat")),
                                         _ptr(out["S0"]), _ptr(ws), ws.numel(), _stream(dev))
        _check(rc, "pic_segment_build_split")
    else:
        ws_n = lib.pic_segment_build_workspace(form, B, H, dk, dv, N, n_seg)
        ws = _workspace(ws_n, dev)
        rc = lib.pic_segment_build(form, dt, precision, B, H, dk, dv, N, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(alpha), _ptr(beta), offs_p, n_seg, _ptr(out["log_scale"]),
                                   _ptr(out.get("T_hat")), _ptr(out["S0"]), _ptr(ws), ws.numel(),
                                   _stream(dev))
        _check(rc, "pic_segment_build")
    if check_finite and precision == PREC_FP16:
        pic_nonfinite_check(dev)
    return out


def pic_segment_prefill(q, k, v, alpha, beta, seg_offsets, *, track_T: bool = True, out=None,
                        check_finite: bool = False):
    """Independent prefill of every segment with per-token outputs (dense
    form, bf16 q/k/v, fp16 operand precision): o_t = S_t^T q_t from the zero
    state at each segment's start, plus the segment's pair.

    q, k: bf16 [B, N, H, dk]; v: bf16 [B, N, H, dv]; alpha, beta: fp32
    [B, N, H] (beta may be None = 1); seg_offsets: host ints [n_seg+1].
    Returns dict: log_scale [n_seg, B, H], S0 [n_seg, B, H, dk, dv], O bf16
    [B, N, H, dv] and, with track_T, T_hat [n_seg, B, H, dk, dk].
    check_finite: wait for the stream and raise PicError when an fp16
    operand overflowed (see pic_nonfinite_check)."""
    lib = load()
    B, N, H, dk = k.shape
    dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16)
    _need(alpha, "alpha", torch.float32)
    _need(beta, "beta", torch.float32)
    if tuple(q.shape) != tuple(k.shape):
        raise ValueError("q must have k's shape")
    off, off_p = _host_i64(seg_offsets)
    n_seg = len(off) - 1
    dev = k.device
    if out is None:
        out = {"log_scale": torch.empty((n_seg, B, H), dtype=torch.float32, device=dev),
               "S0": torch.empty((n_seg, B, H, dk, dv), dtype=torch.float32, device=dev),
               "O": torch.empty((B, N, H, dv), dtype=torch.bfloat16, device=dev)}
        if track_T:
            out["T_hat"] = torch.empty((n_seg, B, H, dk, dk), dtype=torch.float32, device=dev)
    _need(out["log_scale"], "log_scale", torch.float32)
    _need(out["S0"], "S0", torch.float32)
    _need(out["O"], "O", torch.bfloat16)
    if tuple(out["O"].shape) != (B, N, H, dv):
        raise ValueError(f"O must be {(B, N, H, dv)}")
    T = out.get("T_hat")
    _need(T, "T_hat", torch.float32)
    ws = _workspace(lib.pic_segment_build_workspace(FORM_DENSE, B, H, dk, dv, N, n_seg), dev)
    rc = lib.pic_segment_prefill(B, H, dk, dv, N, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                 _ptr(beta), off_p, n_seg, _ptr(out["log_scale"]), _ptr(T),
                                 _ptr(out["S0"]), _ptr(out["O"]), _ptr(ws), ws.numel(),
                                 _stream(dev))
    _check(rc, "pic_segment_prefill")
    if check_finite:
        pic_nonfinite_check(dev)
    return out


def pic_nonfinite_check(device=None):
    """Wait for the device's current stream, then raise PicError
    (PIC_ERR_NONFINITE) if an fp16-operand build or prefill since the last
    check stored a value that is not finite; clears the device's flag."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    _check(load().pic_nonfinite_check(_stream(dev)), "pic_nonfinite_check")


def pic_compose(form: int, pool_log_scale, pool_T_hat, pool_S0, chain_offsets, chain_idx,
                S_in=None, *, out=None, want_pair: bool = False):
    """Fold chains of pool pairs into states: S <- e^lam That S + S0 per step.

    pool_S0: [P, B, H, dk, dv]; pool_log_scale [P, B, H] (diag [P, B, H, dk]);
    pool_T_hat [P, B, H, dk, dk] (dense and KDA; None otherwise).  Returns S_out
    [R, B, H, dk, dv] (``out`` may be S_in for an in-place update).  With
    ``want_pair`` returns (S_out, log_scale_out, T_hat_out): the chain's own
    operator, sum of log scales and (dense) That_pn ... That_p1, else None."""
    lib = load()
    P, B, H, dk, dv = pool_S0.shape
    for t, n in ((pool_log_scale, "pool_log_scale"), (pool_T_hat, "pool_T_hat"),
                 (pool_S0, "pool_S0"), (S_in, "S_in"), (out, "out")):
        _need(t, n, torch.float32)
    off, off_p = _host_i64(chain_offsets)
    idx, idx_p = _host_i32(chain_idx)
    R = len(off) - 1
    dev = pool_S0.device
    if out is None:
        out = torch.empty((R, B, H, dk, dv), dtype=torch.float32, device=dev)
    lam_out = T_out = None
    if want_pair:
        lam_out = torch.empty((R,) + tuple(pool_log_scale.shape[1:]), dtype=torch.float32,
                              device=dev)
        if form in _HAS_T_HAT:
            T_out = torch.empty((R, B, H, dk, dk), dtype=torch.float32, device=dev)
    ws = _workspace(lib.pic_compose_workspace(R, int(off[-1])), dev)
    rc = lib.pic_compose(form, B, H, dk, dv, P, _ptr(pool_log_scale), _ptr(pool_T_hat),
                         _ptr(pool_S0), R, off_p, idx_p, _ptr(S_in), _ptr(out), _ptr(lam_out),
                         _ptr(T_out), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "pic_compose")
    if want_pair:
        return out, lam_out, T_out
    return out


def pic_compose_noalloc(form: int, pool_log_scale, pool_T_hat, pool_S0, chain_offsets,
                        chain_idx, S_in=None, *, out=None, want_pair: bool = False):
    """``pic_compose`` through the library's static scratch: no workspace and
    no allocation inside the call (the outputs are allocated here unless
    given).  Calls that overlap on one device race on the scratch."""
    lib = load()
    P, B, H, dk, dv = pool_S0.shape
    for t, n in ((pool_log_scale, "pool_log_scale"), (pool_T_hat, "pool_T_hat"),
                 (pool_S0, "pool_S0"), (S_in, "S_in"), (out, "out")):
        _need(t, n, torch.float32)
    off, off_p = _host_i64(chain_offsets)
    idx, idx_p = _host_i32(chain_idx)
    R = len(off) - 1
    dev = pool_S0.device
    if out is None:
        out = torch.empty((R, B, H, dk, dv), dtype=torch.float32, device=dev)
    lam_out = T_out = None
    if want_pair:
        lam_out = torch.empty((R,) + tuple(pool_log_scale.shape[1:]), dtype=torch.float32,
                              device=dev)
        if form in _HAS_T_HAT:
            T_out = torch.empty((R, B, H, dk, dk), dtype=torch.float32, device=dev)
    rc = lib.pic_compose_noalloc(form, B, H, dk, dv, P, _ptr(pool_log_scale), _ptr(pool_T_hat),
                                 _ptr(pool_S0), R, off_p, idx_p, _ptr(S_in), _ptr(out),
                                 _ptr(lam_out), _ptr(T_out), _stream(dev))
    _check(rc, "pic_compose_noalloc")
    if want_pair:
        return out, lam_out, T_out
    return out


def pic_naive_add(pool_S0, chain_offsets, chain_idx, S_in=None, *, out=None):
    """The ablation: S_out = S_in + sum of the chain's S0 (no operator)."""
    lib = load()
    P, B, H, dk, dv = pool_S0.shape
    for t, n in ((pool_S0, "pool_S0"), (S_in, "S_in"), (out, "out")):
        _need(t, n, torch.float32)
    off, off_p = _host_i64(chain_offsets)
    idx, idx_p = _host_i32(chain_idx)
    R = len(off) - 1
    dev = pool_S0.device
    if out is None:
        out = torch.empty((R, B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = _workspace(lib.pic_compose_workspace(R, int(off[-1])), dev)
    rc = lib.pic_naive_add(B, H, dk, dv, P, _ptr(pool_S0), R, off_p, idx_p, _ptr(S_in),
                           _ptr(out), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "pic_naive_add")
    return out


def pic_compose_seams(form: int, pool_log_scale, pool_T_hat, pool_S0, chain_offsets, chain_idx,
                      seam_offsets, q, k, v, alpha, beta=None, S_in=None, *, out=None,
                      out_O=None):
    """Reuse with seam windows: each chain entry first runs its seam tokens
    [seam_offsets[c], seam_offsets[c+1]) through the state (writing
    O[t] = S^T q_t after each token), then applies its pair.

    Pool and chains as in ``pic_compose``; q, k: [B, NS, H, dk], v: [B, NS, H, dv]
    (all bf16 or all fp32); alpha fp32 [B, NS, H] (diag [B, NS, H, dk]); beta
    fp32 [B, NS, H] or None (dense only).  Returns (S_out [R, B, H, dk, dv],
    O [B, NS, H, dv])."""
    lib = load()
    P, B, H, dk, dv = pool_S0.shape
    for t, n in ((pool_log_scale, "pool_log_scale"), (pool_T_hat, "pool_T_hat"),
                 (pool_S0, "pool_S0"), (S_in, "S_in"), (out, "out"), (alpha, "alpha"),
                 (beta, "beta"), (out_O, "out_O")):
        _need(t, n, torch.float32)
    if not (q.dtype == k.dtype == v.dtype) or k.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k and v must all be bfloat16 or all float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, None)
    dt = DT_BF16 if k.dtype == torch.bfloat16 else DT_F32
    NS = k.shape[1]
    off, off_p = _host_i64(chain_offsets)
    idx, idx_p = _host_i32(chain_idx)
    soff, soff_p = _host_i64(seam_offsets)
    R = len(off) - 1
    dev = pool_S0.device
    if out is None:
        out = torch.empty((R, B, H, dk, dv), dtype=torch.float32, device=dev)
    if out_O is None:
        out_O = torch.empty((B, NS, H, dv), dtype=torch.float32, device=dev)
    ws = _workspace(lib.pic_compose_seams_workspace(R, int(off[-1])), dev)
    rc = lib.pic_compose_seams(form, dt, B, H, dk, dv, P, _ptr(pool_log_scale),
                               _ptr(pool_T_hat), _ptr(pool_S0), R, off_p, idx_p, soff_p, NS,
                               _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S_in),
                               _ptr(out), _ptr(out_O), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "pic_compose_seams")
    return out, out_O


def pic_rerotate(form: int, pool_log_scale, pool_T_hat, pool_S0, idx, shift, rot_dim: int,
                 base: float = 10000.0, pairing: int = 0, *, out=None):
    """Pool entries idx[j] moved by shift[j] positions under rotary embeddings
    on the keys: S0' = R S0, That' = R That R^T, lambda unchanged (R turns
    channel pair i by shift * base^(-2i/rot_dim); pairing ROPE_INTERLEAVED
    (2i, 2i+1) or ROPE_HALF (i, i + rot_dim/2)).  Returns dict(log_scale,
    T_hat (dense and KDA), S0) with n = len(idx) entries."""
    lib = load()
    P, B, H, dk, dv = pool_S0.shape
    for t, n in ((pool_log_scale, "pool_log_scale"), (pool_T_hat, "pool_T_hat"),
                 (pool_S0, "pool_S0")):
        _need(t, n, torch.float32)
    n_out = len(idx)
    if len(shift) != n_out:
        raise ValueError("idx and shift must have the same length")
    ix, ix_p = _host_i32(idx)
    sh, sh_p = _host_i64(shift)
    dev = pool_S0.device
    if out is None:
        out = {"log_scale": torch.empty((n_out,) + tuple(pool_log_scale.shape[1:]),
                                        dtype=torch.float32, device=dev),
               "S0": torch.empty((n_out, B, H, dk, dv), dtype=torch.float32, device=dev)}
        if form in _HAS_T_HAT:
            out["T_hat"] = torch.empty((n_out, B, H, dk, dk), dtype=torch.float32, device=dev)
    ws = _workspace(lib.pic_rerotate_workspace(n_out), dev)
    rc = lib.pic_rerotate(form, B, H, dk, dv, P, _ptr(pool_log_scale), _ptr(pool_T_hat),
                          _ptr(pool_S0), n_out, ix_p, sh_p, int(rot_dim), float(base),
                          int(pairing), _ptr(out["log_scale"]), _ptr(out.get("T_hat")),
                          _ptr(out["S0"]), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "pic_rerotate")
    return out


def pic_conv_warmup(weight, x, head_start, hist_end, hist_len, n_warm: int, *, out=None):
    """Conv outputs y_t = sum_j weight[..., j] x_(t-j) of the first n_warm tokens
    of each entry's segment, with the previous segment's raw tail as history.

    weight fp32 [H, dc, W]; x [B, N, H, dc] (bf16 or fp32, raw inputs);
    head_start, hist_end: host ints [n]; hist_len: host ints [n] in [0, W-1].
    Returns y [B, n * n_warm, H, dc] in x's dtype (the seam layout)."""
    lib = load()
    B, N, H, dc = x.shape
    W = weight.shape[-1]
    _need(weight, "weight", torch.float32)
    _need(x, "x", None)
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bfloat16 or float32")
    dt = DT_BF16 if x.dtype == torch.bfloat16 else DT_F32
    n = len(head_start)
    if len(hist_end) != n or len(hist_len) != n:
        raise ValueError("head_start, hist_end and hist_len must have the same length")
    hs, hs_p = _host_i64(head_start)
    he, he_p = _host_i64(hist_end)
    hl, hl_p = _host_i32(hist_len)
    shape = (B, n * int(n_warm), H, dc)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    else:
        _need(out, "out", x.dtype)
        if tuple(out.shape) != shape or out.device != x.device:
            raise ValueError(f"out must be {shape} on {x.device}, got {tuple(out.shape)} on "
                             f"{out.device}")
    ws = _workspace(lib.pic_conv_warmup_workspace(n), x.device)
    rc = lib.pic_conv_warmup(dt, B, H, dc, W, N, _ptr(weight), _ptr(x), n, int(n_warm), hs_p,
                             he_p, hl_p, _ptr(out), _ptr(ws), ws.numel(), _stream(x.device))
    _check(rc, "pic_conv_warmup")
    return out


def pic_staging_reserve():
    """Opt into the pinned host pool (current device) for large plan tables,
    so that calls with such tables do not wait for their stream."""
    _check(load().pic_staging_reserve(), "pic_staging_reserve")


def pic_staging_release():
    """Free every pinned staging pool (after their pending copies)."""
    _check(load().pic_staging_release(), "pic_staging_release")


def pic_staging_bytes() -> int:
    """Pinned host bytes the library holds now (0 unless reserved)."""
    return int(load().pic_staging_bytes())


def pic_materialize_T(form: int, log_scale, T_hat=None, dk: int | None = None):
    """Plain fp32 operators T_C = e^lam That for every unit of log_scale."""
    lib = load()
    if form == FORM_DIAG:
        dk = log_scale.shape[-1]
        lead = log_scale.shape[:-1]
    elif form in _HAS_T_HAT:
        dk = T_hat.shape[-1]
        lead = log_scale.shape
    else:
        if dk is None:
            raise ValueError("dk is required for the scalar form")
        lead = log_scale.shape
    _need(log_scale, "log_scale", torch.float32)
    _need(T_hat, "T_hat", torch.float32)
    n_units = 1
    for s in lead:
        n_units *= int(s)
    out = torch.empty(tuple(lead) + (dk, dk), dtype=torch.float32, device=log_scale.device)
    rc = lib.pic_materialize_T(form, n_units, dk, _ptr(log_scale), _ptr(T_hat), _ptr(out),
                               _stream(log_scale.device))
    _check(rc, "pic_materialize_T")
    return out


def pic_split_plan(seg_offsets, n_split: int):
    """The pieces of the split build (pure host code): (piece_offsets [P+1],
    seg_pieces [n_seg+1]) as int64 numpy arrays."""
    lib = load()
    off, off_p = _host_i64(seg_offsets)
    n_seg = len(off) - 1
    n_p = ctypes.c_int64(0)
    seg_p = np.zeros(n_seg + 1, dtype=np.int64)
    cap = n_seg * max(int(n_split), 1) + 1
    pieces = np.zeros(cap, dtype=np.int64)
    rc = lib.pic_split_plan(n_seg, off_p, int(off[-1]) if n_seg >= 0 else 0, int(n_split),
                            pieces.ctypes.data_as(ctypes.c_void_p), cap,
                            seg_p.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n_p))
    _check(rc, "pic_split_plan")
    return pieces[:n_p.value + 1], seg_p


def pic_plan_dump(kind: int, offsets, chain_idx=None, limit: int = 0):
    """Host bookkeeping of a build (kind PLAN_BUILD: rows {segment, start,
    length, n_chunks, tail} in visiting order; limit = n_tokens) or of a
    compose (PLAN_COMPOSE: rows {request, step, pool index}; limit =
    pool_size).  Pure host code; returns an int64 numpy array."""
    lib = load()
    off, off_p = _host_i64(offsets)
    n = len(off) - 1
    if kind == PLAN_BUILD:
        rows, cols = n, PLAN_BUILD_COLS
        idx_p = None
    else:
        rows, cols = int(off[-1]), PLAN_COMPOSE_COLS
        _, idx_p = _host_i32(chain_idx)
    table = np.zeros((max(rows, 1), cols), dtype=np.int64)
    rc = lib.pic_plan_dump(kind, n, off_p, idx_p, int(limit),
                           table.ctypes.data_as(ctypes.c_void_p), rows)
    _check(rc, "pic_plan_dump")
    return table[:rows]
