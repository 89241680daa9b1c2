"""fp64 CPU oracle of the linear-attention segment transform (HYPIC).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``hybrid_caching_amd``) never imports it, and the two share no code.

The arithmetic lives in ``pic_oracle.c`` (plain C, fp64, plain loops); this
module only marshals numpy arrays into it.  What each call computes:

* ``build``      -- per (segment, layer, head): lambda_C = sum ln(alpha),
  That_C = prod (I - beta k k^T) (dense), plain T_C and S(C|0) from a zero
  state.  [xix.ai HYPIC article (French), paragraph on linear layers: the
  accumulated transition operator T_C and the zero-start final state S(C|0)]
* ``recurrence`` -- the unsplit per-token recurrence from S_in.
* ``compose``    -- S <- T_C S + S(C|0) along a chain of cached pairs.
  [same paragraph: left-multiply by T_C, then add]
* ``naive_add``  -- S_in + sum S(C|0), the ablation.  [same paragraph]
* ``seam_compose`` -- reuse with seam windows: before each cached pair, the
  entry's seam tokens advance the state one token at a time and each emits
  o_t = S_t^T q_t.  [xix.ai, paragraph on full-attention layers: the first w
  tokens of every inner segment are left out of the cache and recomputed on
  reuse; linear layers advance the running state through them and pass each
  token's output up]
* ``rope_matrix`` / ``rerotate`` -- moving a cached pair to another position
  under rotary position embeddings on the keys: with R_p the rotation of
  offset p, S' = R_p S and That' = R_p That R_p^T (lambda unchanged), written
  as explicit fp64 matrices and matrix products (numpy).  [xix.ai, paragraph
  on linear layers: variants with rotary embeddings need the cached state
  re-rotated]
* ``conv_warmup`` -- the first tokens of a segment under a short causal
  depthwise convolution of width W, recomputed with the previous segment's
  last raw inputs as history: y_t = sum_j w_j x_(t-j), written as plain loops.
  [xix.ai, paragraph on linear layers: variants with a short convolution need
  the convolution state warmed up]
* ``prefill`` -- the independent prefill of every segment with per-token
  outputs o_t = S_t^T q_t (the state after the token's own update), beside
  the pair: the build's token loop with a readout after every update.
  [remio.ai, section on how HYPIC composes linear-attention states: the pair
  is built at the segment's first prefill]
* ``plan_build`` / ``plan_compose`` -- the host bookkeeping of a call, from
  its definition: segments as token ranges cut into 64-token chunks (in
  segment order; the order a launch visits them in is the library's
  schedule); chains applied entry by entry.  Pinned against hand-written
  tables.

Forms: 0 = scalar decay, 1 = diagonal gate, 2 = dense gated delta (GDN form),
3 = dense delta with per-channel gates (KDA form, T_t = (I - b k k^T) Diag(a)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

SCALAR, DIAG, DENSE, KDA = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pic_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpic_oracle.so")
_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)


def compile_oracle(out_path: str = _LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle's C source with gcc into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", *extra_flags, "-o", out_path, src,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out_path


def _bind(lib):
    lib.oracle_build.restype = ctypes.c_int
    lib.oracle_build.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int64, _dp, _dp, _dp, _dp,
                                 _i64p, ctypes.c_int, _dp, _dp, _dp, _dp, ctypes.c_int]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int64, _dp, _dp, _dp, _dp,
                                   _dp, _i64p, ctypes.c_int, _dp, _dp, _dp, _dp, _dp,
                                   ctypes.c_int]
    lib.oracle_recurrence.restype = ctypes.c_int
    lib.oracle_recurrence.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int64, _dp, _dp, _dp, _dp, _dp, _dp,
                                      ctypes.c_int]
    lib.oracle_compose.restype = ctypes.c_int
    lib.oracle_compose.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int64, _dp, _dp, _dp, ctypes.c_int,
                                   _i64p, _i32p, _dp, _dp, _dp, _dp, ctypes.c_int]
    lib.oracle_seam_compose.restype = ctypes.c_int
    lib.oracle_seam_compose.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int64, _dp, _dp, _dp,
                                        ctypes.c_int, _i64p, _i32p, _i64p, ctypes.c_int64, _dp,
                                        _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
    lib.oracle_naive_add.restype = ctypes.c_int
    lib.oracle_naive_add.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int64, _dp, ctypes.c_int, _i64p, _i32p, _dp, _dp,
                                     ctypes.c_int]
    return lib


def load(path: str | None = None):
    """Load (compiling first if needed) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(_LIB_PATH)
                    or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                compile_oracle()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, t=_dp):
    if a is None:
        return ctypes.cast(None, t)
    return a.ctypes.data_as(t)


def build(form, k, v, alpha, beta, offsets, *, literal=False, want_T=False, threads=None,
          lib=None):
    """Build the pair of every (segment, layer, head).

    k: [B, N, H, dk]; v: [B, N, H, dv]; alpha: [B, N, H] (diag: [B, N, H, dk]);
    beta: [B, N, H] or None (= 1; ignored for scalar/diag); offsets: n_seg+1 ints.
    Returns dict with lam [n_seg, B, H(, dk)], That [n_seg, B, H, dk, dk] (dense),
    T (plain T_C, if want_T or literal) and S [n_seg, B, H, dk, dv], all fp64.
    """
    lib = lib or load()
    k, v, alpha = _f64(k), _f64(v), _f64(alpha)
    beta = _f64(beta) if (beta is not None and form in (DENSE, KDA)) else None
    B, N, H, dk = k.shape
    dv = v.shape[3]
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    n_seg = len(offs) - 1
    lam = np.zeros((n_seg, B, H, dk) if form == DIAG else (n_seg, B, H))
    That = np.zeros((n_seg, B, H, dk, dk)) if form in (DENSE, KDA) else None
    T = np.zeros((n_seg, B, H, dk, dk)) if (want_T or literal) else None
    S = np.zeros((n_seg, B, H, dk, dv))
    rc = lib.oracle_build(form, int(bool(literal)), B, H, dk, dv, N, _ptr(k), _ptr(v),
                          _ptr(alpha), _ptr(beta), _ptr(offs, _i64p), n_seg, _ptr(lam),
                          _ptr(That), _ptr(T), _ptr(S), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_build rejected its arguments")
    out = {"lam": lam, "S": S}
    if That is not None:
        out["That"] = That
    if T is not None:
        out["T"] = T
    return out


def prefill(form, q, k, v, alpha, beta, offsets, *, literal=False, threads=None, lib=None):
    """Independent prefill of every segment with per-token outputs.

    Each segment starts from the zero state; after every token's update
    S_t = T_t S_(t-1) + beta_t k_t v_t^T its output is o_t = S_t^T q_t (the
    readout of the state that includes the token).  q: [B, N, H, dk]; the
    rest as for ``build``.  Returns ``build``'s dict plus O [B, N, H, dv].
    [the pair is cached at a segment's first prefill, alongside the prefill's
    own outputs; remio.ai HYPIC article (Japanese), section on how HYPIC
    composes linear-attention states]"""
    lib = lib or load()
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    beta = _f64(beta) if (beta is not None and form in (DENSE, KDA)) else None
    B, N, H, dk = k.shape
    dv = v.shape[3]
    if q.shape != k.shape:
        raise ValueError("q must have k's shape")
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    n_seg = len(offs) - 1
    lam = np.zeros((n_seg, B, H, dk) if form == DIAG else (n_seg, B, H))
    That = np.zeros((n_seg, B, H, dk, dk)) if form in (DENSE, KDA) else None
    T = np.zeros((n_seg, B, H, dk, dk)) if literal else None
    S = np.zeros((n_seg, B, H, dk, dv))
    O = np.zeros((B, N, H, dv))
    rc = lib.oracle_prefill(form, int(bool(literal)), B, H, dk, dv, N, _ptr(q), _ptr(k), _ptr(v),
                            _ptr(alpha), _ptr(beta), _ptr(offs, _i64p), n_seg, _ptr(lam),
                            _ptr(That), _ptr(T), _ptr(S), _ptr(O), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    out = {"lam": lam, "S": S, "O": O}
    if That is not None:
        out["That"] = That
    if T is not None:
        out["T"] = T
    return out


def recurrence(form, k, v, alpha, beta, S_in=None, *, threads=None, lib=None):
    """Unsplit literal recurrence over all N tokens from S_in: returns [B, H, dk, dv]."""
    lib = lib or load()
    k, v, alpha = _f64(k), _f64(v), _f64(alpha)
    beta = _f64(beta) if (beta is not None and form in (DENSE, KDA)) else None
    B, N, H, dk = k.shape
    dv = v.shape[3]
    S_in = _f64(S_in)
    out = np.zeros((B, H, dk, dv))
    rc = lib.oracle_recurrence(form, B, H, dk, dv, N, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(S_in), _ptr(out), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_recurrence rejected its arguments")
    return out


def _chains(chain_offsets, chain_idx):
    off = np.ascontiguousarray(np.asarray(chain_offsets, dtype=np.int64))
    idx = np.ascontiguousarray(np.asarray(chain_idx, dtype=np.int32))
    if idx.size == 0:
        idx = np.zeros(1, dtype=np.int32)
    return off, idx


def compose(form, lam, That, S, chain_offsets, chain_idx, S_in=None, *, want_pair=False,
            threads=None, lib=None):
    """Compose chains of pool pairs onto S_in.

    Pool: lam [P, B, H(, dk)], That [P, B, H, dk, dk] (dense; None otherwise),
    S [P, B, H, dk, dv].  Request r applies pool entries
    chain_idx[chain_offsets[r]:chain_offsets[r+1]] in order.  Returns S_out
    [R, B, H, dk, dv] (and the chain's own (lam, That) if want_pair).
    """
    lib = lib or load()
    lam, S = _f64(lam), _f64(S)
    That = _f64(That) if form in (DENSE, KDA) else None
    P, B, H, dk, dv = S.shape
    off, idx = _chains(chain_offsets, chain_idx)
    R = len(off) - 1
    S_in = _f64(S_in)
    S_out = np.zeros((R, B, H, dk, dv))
    lam_out = np.zeros((R,) + lam.shape[1:]) if want_pair else None
    That_out = np.zeros((R, B, H, dk, dk)) if (want_pair and form in (DENSE, KDA)) else None
    rc = lib.oracle_compose(form, B, H, dk, dv, P, _ptr(lam), _ptr(That), _ptr(S), R,
                            _ptr(off, _i64p), _ptr(idx, _i32p), _ptr(S_in), _ptr(S_out),
                            _ptr(lam_out), _ptr(That_out), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_compose rejected its arguments")
    if want_pair:
        return S_out, lam_out, That_out
    return S_out


def naive_add(S, chain_offsets, chain_idx, S_in=None, *, threads=None, lib=None):
    """S_in + sum of the chain's zero-start states: returns [R, B, H, dk, dv]."""
    lib = lib or load()
    S = _f64(S)
    P, B, H, dk, dv = S.shape
    off, idx = _chains(chain_offsets, chain_idx)
    R = len(off) - 1
    S_in = _f64(S_in)
    S_out = np.zeros((R, B, H, dk, dv))
    rc = lib.oracle_naive_add(B, H, dk, dv, P, _ptr(S), R, _ptr(off, _i64p), _ptr(idx, _i32p),
                              _ptr(S_in), _ptr(S_out), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_naive_add rejected its arguments")
    return S_out


def seam_compose(form, lam, That, S, chain_offsets, chain_idx, seam_offsets, q, k, v, alpha,
                 beta, S_in=None, *, literal=False, threads=None, lib=None):
    """Reuse with seam windows.

    Pool as in ``compose``.  Chain entry c (over all requests, in order) has
    the seam tokens [seam_offsets[c], seam_offsets[c+1]) of q, k: [B, NS, H, dk],
    v: [B, NS, H, dv], alpha: [B, NS, H] (diag, KDA: [B, NS, H, dk]), beta:
    [B, NS, H] or None (dense, KDA).  Each entry advances the state through its seam tokens (emitting
    o_t = S_t^T q_t) and then applies its pair.  Returns (S_out [R, B, H, dk, dv],
    O [B, NS, H, dv]).
    """
    lib = lib or load()
    lam, S = _f64(lam), _f64(S)
    That = _f64(That) if form in (DENSE, KDA) else None
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    beta = _f64(beta) if (beta is not None and form in (DENSE, KDA)) else None
    P, B, H, dk, dv = S.shape
    NS = k.shape[1]
    off, idx = _chains(chain_offsets, chain_idx)
    soff = np.ascontiguousarray(np.asarray(seam_offsets, dtype=np.int64))
    R = len(off) - 1
    S_in = _f64(S_in)
    S_out = np.zeros((R, B, H, dk, dv))
    O = np.zeros((B, NS, H, dv))
    rc = lib.oracle_seam_compose(form, int(bool(literal)), B, H, dk, dv, P, _ptr(lam), _ptr(That),
                                 _ptr(S), R, _ptr(off, _i64p), _ptr(idx, _i32p), _ptr(soff, _i64p),
                                 NS, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(S_in), _ptr(S_out), _ptr(O), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_seam_compose rejected its arguments")
    return S_out, O


CHUNK = 64


def plan_build(seg_offsets):
    """One row per segment, in segment order: (segment, start, length,
    n_chunks, tail).  Segment s covers tokens [off[s], off[s+1]); it is cut
    into n_chunks = ceil(length / 64) chunks of 64 tokens, the last holding
    tail = length - 64 (n_chunks - 1) tokens (1..64), or none when the segment
    is empty (n_chunks = tail = 0).  The order in which a launch visits the
    segments is the library's schedule, not part of this definition.
    [each segment is a token range found from its boundaries and gets its own
    pair; xix.ai HYPIC article, paragraph on linear layers]"""
    off = [int(x) for x in seg_offsets]
    rows = []
    for s in range(len(off) - 1):
        length = off[s + 1] - off[s]
        n_chunks = (length + CHUNK - 1) // CHUNK
        tail = length - CHUNK * (n_chunks - 1) if n_chunks else 0
        rows.append((s, off[s], length, n_chunks, tail))
    return np.array(rows, dtype=np.int64).reshape(len(rows), 5)


def plan_compose(chain_offsets, chain_idx):
    """One row per chain entry, in application order: (request, step, pool
    index), where request r owns entries [off[r], off[r+1]) and step counts
    from the request's own first entry.  [the cached pairs of a request are
    applied to its running state one after another, in prompt order; xix.ai
    HYPIC article, paragraph on linear layers]"""
    off = [int(x) for x in chain_offsets]
    idx = [int(x) for x in chain_idx]
    rows = [(r, c - off[r], idx[c]) for r in range(len(off) - 1) for c in range(off[r], off[r + 1])]
    return np.array(rows, dtype=np.int64).reshape(len(rows), 3)


# --------------------------------------------------------------------------
# re-rotation of cached pairs (rotary position embeddings on the keys)
# --------------------------------------------------------------------------

ROPE_INTERLEAVED, ROPE_HALF = 0, 1


def rope_matrix(dk, shift, rot_dim, base, pairing=ROPE_INTERLEAVED):
    """The dk x dk rotation R_shift of rotary position embeddings, fp64.

    Channel pair i (i < rot_dim / 2) is (2i, 2i+1) (interleaved) or
    (i, i + rot_dim/2) (half); it turns by the angle shift * base^(-2i/rot_dim):
    (x_a, x_b) -> (cos x_a - sin x_b, sin x_a + cos x_b).  Channels at and past
    rot_dim are left alone.  Keys at position t are R_t k; R_p R_t = R_(p+t)."""
    R = np.eye(dk)
    h = rot_dim // 2
    for i in range(h):
        a, b = (2 * i, 2 * i + 1) if pairing == ROPE_INTERLEAVED else (i, i + h)
        phi = float(shift) * float(base) ** (-2.0 * i / rot_dim)
        c, s = np.cos(phi), np.sin(phi)
        R[a, a], R[a, b], R[b, a], R[b, b] = c, -s, s, c
    return R


def rerotate(form, lam, That, S, idx, shift, rot_dim, base, pairing=ROPE_INTERLEAVED):
    """Pool entries idx[j] moved by shift[j] positions: a segment whose keys
    were rotated at positions t is given keys rotated at positions t + shift.

    Reading: every key gains the factor R_shift, an orthogonal matrix, so each
    token transition becomes R T_t R^T (exactly for the scalar and dense
    forms; for the diagonal and KDA forms only when the gates of the two
    channels of every rotated pair are equal) and by induction
    S(C|0) -> R S(C|0), T_C -> R T_C R^T; lambda is unchanged.
    Returns (lam_out [n, ...], That_out [n, B, H, dk, dk] or None,
    S_out [n, B, H, dk, dv])."""
    lam, S = _f64(lam), _f64(S)
    That = _f64(That) if That is not None else None
    idx = [int(i) for i in idx]
    shift = [int(p) for p in shift]
    dk = S.shape[-2]
    lam_out = np.stack([lam[i] for i in idx]) if idx else np.zeros((0,) + lam.shape[1:])
    S_out = np.zeros((len(idx),) + S.shape[1:])
    T_out = np.zeros((len(idx),) + That.shape[1:]) if That is not None else None
    for j, (i, p) in enumerate(zip(idx, shift)):
        R = rope_matrix(dk, p, rot_dim, base, pairing)
        S_out[j] = np.matmul(R, S[i])
        if That is not None:
            T_out[j] = np.matmul(np.matmul(R, That[i]), R.T)
    return lam_out, T_out, S_out


# --------------------------------------------------------------------------
# convolution warm-up (short causal depthwise convolution before the layer)
# --------------------------------------------------------------------------

def conv_warmup(weight, x, hist_end, hist_len, head_start, n_warm):
    """Conv outputs of the first n_warm tokens of each entry's segment.

    weight [H, dc, W]: y_t = sum_{j < W} weight[..., j] * x_(t-j) per channel
    (j = 0 the token itself).  x [B, N, H, dc] raw inputs.  Entry e reads its
    head tokens x[:, head_start[e] + t] and, for t - j < 0, the history token
    x[:, hist_end[e] + (t - j)] when -(t - j) <= hist_len[e], else 0 (no
    history: the independent prefill).  Returns y [B, n * n_warm, H, dc],
    entry e's tokens at rows e * n_warm .. e * n_warm + n_warm - 1."""
    w = _f64(weight)
    x = _f64(x)
    B, N, H, dc = x.shape
    W = w.shape[-1]
    n = len(head_start)
    y = np.zeros((B, n * n_warm, H, dc))
    for e in range(n):
        for t in range(n_warm):
            acc = np.zeros((B, H, dc))
            for j in range(W):
                tau = t - j
                if tau >= 0:
                    xv = x[:, int(head_start[e]) + tau]
                elif -tau <= int(hist_len[e]):
                    xv = x[:, int(hist_end[e]) + tau]
                else:
                    continue
                acc = acc + w[None, :, :, j] * xv
            y[:, e * n_warm + t] = acc
    return y

