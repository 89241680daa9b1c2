"""The C ABI on the host: the library loads, exports every function declared in
include/pic.h, and its validation (which makes no HIP call) returns the
documented status codes.  Runs without a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pic.h")

OK, ENULL, EDIMS, EOFF, ECHAIN, EWS, EUNSUP, EHIP, EALIGN = 0, -1, -2, -3, -4, -5, -6, -7, -8
SCALAR, DIAG, DENSE, KDA = 0, 1, 2, 3
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    from hybrid_caching_amd import _build, _lib
    if not os.path.exists(_lib.LIB_PATH):
        _build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pic_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("pic_segment_build", "pic_compose", "pic_naive_add", "pic_validate_build",
              "pic_validate_compose", "pic_validate_naive_add", "pic_materialize_T",
              "pic_last_error", "pic_status_string", "pic_abi_version",
              "pic_segment_build_workspace", "pic_compose_workspace", "pic_plan_dump",
              "pic_compose_seams", "pic_validate_compose_seams", "pic_compose_seams_workspace"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from hybrid_caching_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def test_version_and_status_strings(lib):
    assert lib.pic_abi_version() == 11
    for code in (OK, ENULL, EDIMS, EOFF, ECHAIN, EWS, EUNSUP, EHIP, EALIGN, -9):
        s = lib.pic_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.pic_status_string(12345).decode() == "unknown status"


# fake, aligned device addresses: validation never dereferences them
A = 0x10000


def P(i):
    return ctypes.c_void_p(A * (i + 1))


def offsets(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def vbuild(lib, form=DENSE, dt=BF16, B=1, H=2, dk=128, dv=128, N=100, offs=(0, 40, 100),
           That=True, ws_bytes=None, k=None, alpha=None, S0=None, ws=None, prec=0):
    off, off_p = offsets(offs)
    n_seg = len(off) - 1
    need = lib.pic_segment_build_workspace(form, B, H, dk, dv, N, n_seg)
    return lib.pic_validate_build(form, dt, prec, B, H, dk, dv, N, None, k or P(0), P(1),
                                  alpha or P(2), P(3), off_p, n_seg, P(4),
                                  P(5) if That else None, S0 or P(6), ws or P(7),
                                  need if ws_bytes is None else ws_bytes)


def test_validate_build_accepts_good_arguments(lib):
    assert vbuild(lib) == OK
    assert vbuild(lib, form=SCALAR, That=False) == OK
    assert vbuild(lib, form=DIAG, That=False, dt=F32, dk=16, dv=48) == OK
    assert vbuild(lib, offs=(0, 0, 100, 100)) == OK  # empty segments are allowed
    assert vbuild(lib, prec=1) == OK  # fp16 operands: dense with bf16 k/v
    assert vbuild(lib, prec=1, dk=16, dv=48) == OK
    assert vbuild(lib, form=KDA) == OK  # per-channel gates, That required
    assert vbuild(lib, form=KDA, dt=F32, dk=32, dv=96) == OK
    assert vbuild(lib, form=KDA, prec=1) == OK  # chunked: bf16 k/v, dk = dv = 128
    assert lib.pic_last_error().decode() == ""


@pytest.mark.parametrize("kw,code", [
    ({"form": 7}, EUNSUP), ({"dt": 5}, EUNSUP), ({"prec": 2}, EUNSUP), ({"prec": -1}, EUNSUP),
    ({"prec": 1, "dt": F32}, EUNSUP), ({"prec": 1, "form": SCALAR, "That": False}, EUNSUP),
    ({"prec": 1, "form": DIAG, "That": False}, EUNSUP),
    ({"prec": 1, "form": KDA, "dk": 64, "dv": 64}, EUNSUP),
    ({"prec": 1, "form": KDA, "dv": 64}, EUNSUP), ({"prec": 1, "form": KDA, "dt": F32}, EUNSUP),
    ({"form": KDA, "That": False}, ENULL), ({"form": 4}, EUNSUP),
    ({"dk": 8}, EDIMS), ({"dv": 144}, EDIMS), ({"dk": 24}, EDIMS), ({"B": 0}, EDIMS),
    ({"H": 0}, EDIMS),
    ({"offs": (1, 40, 100)}, EOFF), ({"offs": (0, 50, 40, 100)}, EOFF),
    ({"offs": (0, 40, 99)}, EOFF), ({"offs": (0, 40, 101)}, EOFF),
    ({"That": False}, ENULL), ({"form": SCALAR, "That": True}, EUNSUP),
    ({"ws_bytes": 8}, EWS),
    ({"k": ctypes.c_void_p(A + 4)}, EALIGN), ({"S0": ctypes.c_void_p(A + 8)}, EALIGN),
])
def test_validate_build_rejects(lib, kw, code):
    assert vbuild(lib, **kw) == code
    assert lib.pic_last_error().decode() != ""


def test_validate_build_null_pointers(lib):
    off, off_p = offsets((0, 10))
    ws = lib.pic_segment_build_workspace(DENSE, 1, 1, 16, 16, 10, 1)
    args = [DENSE, BF16, 0, 1, 1, 16, 16, 10, None, P(0), P(1), P(2), None, off_p, 1, P(4),
            P(5), P(6), P(7), ws]
    assert lib.pic_validate_build(*args) == OK
    for i in (9, 10, 11, 13, 15, 16, 17, 18):  # k, v, alpha, offsets, lam, That, S0, workspace
        bad = list(args)
        bad[i] = None
        rc = lib.pic_validate_build(*bad)
        assert rc in (ENULL, EWS), (i, rc)


def vprefill(lib, B=1, H=2, dk=128, dv=128, N=100, offs=(0, 40, 100), That=True, O=True,
             ws_bytes=None, q=None, O_ptr=None):
    off, off_p = offsets(offs)
    n_seg = len(off) - 1
    need = lib.pic_segment_build_workspace(DENSE, B, H, dk, dv, N, n_seg)
    return lib.pic_validate_prefill(B, H, dk, dv, N, q or P(8), P(0), P(1), P(2), P(3), off_p,
                                    n_seg, P(4), P(5) if That else None, P(6),
                                    (O_ptr or P(9)) if O else None, P(7),
                                    need if ws_bytes is None else ws_bytes)


def test_validate_prefill(lib):
    assert vprefill(lib) == OK
    assert vprefill(lib, That=False) == OK  # That is optional: the plain prefill
    assert vprefill(lib, dk=16, dv=48, offs=(0, 0, 100)) == OK
    assert vprefill(lib, O=False) == ENULL
    assert vprefill(lib, q=None, O=True) == OK
    assert vprefill(lib, dk=24) == EDIMS
    assert vprefill(lib, offs=(0, 40, 99)) == EOFF
    assert vprefill(lib, ws_bytes=8, offs=tuple(range(0, 101, 2))) == EWS
    assert vprefill(lib, O_ptr=ctypes.c_void_p(A + 9 * 4096 + 2)) == EALIGN
    # outputs overlapping an input are refused (k lies at A + 4096)
    assert vprefill(lib, O_ptr=ctypes.c_void_p(A + 4096)) == EUNSUP
    assert lib.pic_last_error().decode() != ""


def vcompose(lib, form=DENSE, B=1, H=2, dk=128, dv=128, pool=5, off=(0, 3, 3, 5),
             idx=(4, 0, 1, 2, 3), That=True, ws_bytes=None, S_in=None, lam_out=None,
             T_out=None):
    o, o_p = offsets(off)
    i = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    i_p = i.ctypes.data_as(ctypes.c_void_p) if i.size else None
    R = len(o) - 1
    need = lib.pic_compose_workspace(R, int(o[-1]))
    return lib.pic_validate_compose(form, B, H, dk, dv, pool, P(0), P(1) if That else None,
                                    P(2), R, o_p, i_p, S_in or P(3), P(4), lam_out, T_out,
                                    P(5), need if ws_bytes is None else ws_bytes)


def test_validate_compose(lib):
    assert vcompose(lib) == OK
    assert vcompose(lib, form=SCALAR, That=False) == OK
    assert vcompose(lib, off=(0, 0), idx=()) == OK  # one empty chain
    assert vcompose(lib, off=(0,), idx=()) == OK  # no requests
    assert vcompose(lib, idx=(4, 0, 1, 2, 5)) == ECHAIN
    assert vcompose(lib, idx=(4, 0, -1, 2, 3)) == ECHAIN
    assert vcompose(lib, off=(1, 3, 3, 5)) == ECHAIN
    assert vcompose(lib, off=(0, 3, 2, 5)) == ECHAIN
    assert vcompose(lib, That=False) == ENULL
    assert vcompose(lib, form=DIAG, That=True) == EUNSUP
    assert vcompose(lib, form=KDA) == OK  # KDA pairs compose like dense ones
    assert vcompose(lib, form=KDA, That=False) == ENULL
    assert vcompose(lib, form=4) == EUNSUP
    assert vcompose(lib, ws_bytes=1) == EWS
    assert vcompose(lib, dk=130) == EDIMS
    assert vcompose(lib, S_in=ctypes.c_void_p(A + 2)) == EALIGN


def test_validate_compose_chain_pair(lib):
    """The chain's own pair: dense needs log_scale_out and T_hat_out together;
    the other forms take log_scale_out only."""
    assert vcompose(lib, lam_out=P(6), T_out=P(7)) == OK
    assert vcompose(lib, lam_out=P(6)) == ENULL
    assert vcompose(lib, T_out=P(7)) == ENULL
    assert vcompose(lib, form=SCALAR, That=False, lam_out=P(6)) == OK
    assert vcompose(lib, form=DIAG, That=False, lam_out=P(6)) == OK
    assert vcompose(lib, form=KDA, lam_out=P(6), T_out=P(7)) == OK
    assert vcompose(lib, form=KDA, lam_out=P(6)) == ENULL
    assert vcompose(lib, form=SCALAR, That=False, lam_out=P(6), T_out=P(7)) == EUNSUP
    assert vcompose(lib, lam_out=P(6), T_out=ctypes.c_void_p(A + 6 * 4096 + 4)) == EALIGN


# --------------------------------------------------------------------------
# plan dump: exact bookkeeping against the oracle's definition of the plan
# --------------------------------------------------------------------------

def _plan_cases():
    rng = np.random.default_rng(5)
    cases = [[0, 64], [0, 0], [0, 63, 127, 127, 300, 364], [0, 1, 2, 3], [0, 4096] * 1]
    for _ in range(20):
        n = int(rng.integers(1, 40))
        lens = rng.choice([0, 1, 63, 64, 65, 128, 200, 4096], size=n)
        cases.append([0] + list(np.cumsum(lens)))
    return cases


def test_build_plan_matches_oracle_plan():
    """The library's rows are the oracle's rows (per segment), in the
    library's visiting order: longest segment first, ties by lower index (a
    schedule, checked here as a property of the library, not of the method)."""
    import oracle
    from hybrid_caching_amd import _lib
    for off in _plan_cases():
        got = _lib.pic_plan_dump(_lib.PLAN_BUILD, off, limit=off[-1])
        ref = oracle.plan_build(off)
        assert got.dtype == np.int64 and got.shape == ref.shape, off
        assert np.array_equal(got[np.argsort(got[:, 0], kind="stable")], ref), off
        assert sorted(got[:, 0].tolist()) == list(range(len(off) - 1)), off
        key = [(-int(r[2]), int(r[0])) for r in got]
        assert key == sorted(key), off


def test_compose_plan_matches_oracle_plan():
    import oracle
    from hybrid_caching_amd import _lib
    rng = np.random.default_rng(6)
    for R in (0, 1, 5, 64):
        lens = rng.integers(0, 60, size=R)
        off = [0] + list(np.cumsum(lens))
        idx = rng.integers(0, 256, size=int(off[-1]))
        got = _lib.pic_plan_dump(_lib.PLAN_COMPOSE, off, idx, limit=256)
        ref = oracle.plan_compose(off, idx)
        assert np.array_equal(got, ref), R


def test_plan_dump_errors(lib):
    o, o_p = offsets((0, 10, 5))
    table = np.zeros((4, 5), dtype=np.int64)
    t_p = table.ctypes.data_as(ctypes.c_void_p)
    assert lib.pic_plan_dump(0, 2, o_p, None, 5, t_p, 4) == EOFF
    o, o_p = offsets((0, 10, 20))
    assert lib.pic_plan_dump(0, 2, o_p, None, 21, t_p, 4) == EOFF   # last != n_tokens
    assert lib.pic_plan_dump(0, 2, o_p, None, 20, t_p, 1) == EWS    # table too small
    assert lib.pic_plan_dump(0, 2, o_p, None, 20, None, 4) == ENULL
    assert lib.pic_plan_dump(0, 2, o_p, None, 20, t_p, 4) == OK
    assert table[0].tolist() == [0, 0, 10, 1, 10] and table[1].tolist() == [1, 10, 10, 1, 10]
    assert lib.pic_plan_dump(7, 2, o_p, None, 20, t_p, 4) == EUNSUP
    i = np.array([0, 3], dtype=np.int32)
    c, c_p = offsets((0, 2))
    assert lib.pic_plan_dump(1, 1, c_p, i.ctypes.data_as(ctypes.c_void_p), 3, t_p, 4) == ECHAIN


def test_no_memory_is_held_by_default(lib):
    """The library holds no pinned memory unless the caller reserves it."""
    assert lib.pic_staging_bytes() == 0


def test_validate_naive_add(lib):
    o, o_p = offsets((0, 2))
    i = np.array([1, 0], dtype=np.int32)
    need = lib.pic_compose_workspace(1, 2)
    args = [1, 2, 64, 64, 2, P(0), 1, o_p, i.ctypes.data_as(ctypes.c_void_p), None, P(1), P(2),
            need]
    assert lib.pic_validate_naive_add(*args) == OK
    bad = list(args)
    bad[4] = 1  # pool of one: index 1 out of range
    assert lib.pic_validate_naive_add(*bad) == ECHAIN
    bad = list(args)
    bad[12] = 0
    assert lib.pic_validate_naive_add(*bad) == EWS


def test_workspace_queries_grow_with_the_plan(lib):
    a = lib.pic_segment_build_workspace(DENSE, 1, 1, 128, 128, 100, 4)
    b = lib.pic_segment_build_workspace(DENSE, 1, 1, 128, 128, 100, 4000)
    assert 0 < a < b
    assert 0 < lib.pic_compose_workspace(1, 4) < lib.pic_compose_workspace(64, 100000)


def test_product_path_does_not_import_the_oracle():
    """The HIP path and the oracle share no code and neither imports the other."""
    pkg = os.path.join(ROOT, "hybrid_caching_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "pic_oracle" not in text, f
    src = open(os.path.join(ROOT, "oracle", "pic_oracle.c"), encoding="utf-8").read()
    assert "pic.h" not in src and "hybrid_caching_amd" not in src


def vseams(lib, form=DENSE, dt=BF16, B=1, H=2, dk=128, dv=128, pool=5, off=(0, 3, 3, 5),
           idx=(4, 0, 1, 2, 3), seam=(0, 0, 8, 16, 16, 20), That=True, ws_bytes=None,
           q=None, O=None, beta=None, n_seam=None):
    o, o_p = offsets(off)
    i = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    i_p = i.ctypes.data_as(ctypes.c_void_p) if i.size else None
    so, so_p = offsets(seam)
    R = len(o) - 1
    ns = int(so[-1]) if n_seam is None else n_seam
    need = lib.pic_compose_seams_workspace(R, int(o[-1]))
    return lib.pic_validate_compose_seams(
        form, dt, B, H, dk, dv, pool, P(0), P(1) if That else None, P(2), R, o_p, i_p, so_p, ns,
        P(6) if q is None else q, P(7), P(8), P(9), beta, P(3), P(4),
        P(10) if O is None else O, P(5),
        need if ws_bytes is None else ws_bytes)


def test_validate_compose_seams(lib):
    assert vseams(lib) == OK
    assert vseams(lib, form=SCALAR, That=False, dt=F32) == OK
    assert vseams(lib, form=DIAG, That=False, dk=16, dv=64) == OK
    assert vseams(lib, beta=P(11)) == OK
    assert vseams(lib, seam=(0, 0, 0, 0, 0, 0)) == OK  # no seam tokens at all
    assert vseams(lib, seam=(0, 0, 0, 0, 0, 0), q=ctypes.c_void_p(0), O=ctypes.c_void_p(0)) == OK
    assert vseams(lib, off=(0,), idx=(), seam=(0,)) == OK
    assert vseams(lib, seam=(0, 64, 64, 64, 64, 64)) == OK  # the largest window
    assert vseams(lib, form=KDA) == OK  # KDA seams: per-channel gates, That required
    assert lib.pic_last_error().decode() == ""


@pytest.mark.parametrize("kw,code", [
    ({"form": KDA, "That": False}, ENULL), ({"form": 4}, EUNSUP), ({"dt": 2}, EUNSUP),
    ({"dk": 8}, EDIMS),
    ({"seam": (1, 1, 8, 16, 16, 20)}, EOFF), ({"seam": (0, 8, 4, 16, 16, 20)}, EOFF),
    ({"seam": (0, 0, 8, 16, 16, 20), "n_seam": 21}, EOFF),
    ({"seam": (0, 65, 65, 65, 65, 65)}, EDIMS), ({"n_seam": -1}, EDIMS),
    ({"idx": (4, 0, 1, 2, 9)}, ECHAIN), ({"That": False}, ENULL),
    ({"form": SCALAR, "That": True}, EUNSUP),
    ({"q": ctypes.c_void_p(0)}, ENULL), ({"O": ctypes.c_void_p(0)}, ENULL),
    ({"ws_bytes": 8}, EWS), ({"q": ctypes.c_void_p(A + 2)}, EALIGN),
])
def test_validate_compose_seams_rejects(lib, kw, code):
    assert vseams(lib, **kw) == code
    assert lib.pic_last_error().decode() != ""


def test_compose_seams_workspace_grows_with_the_chain(lib):
    assert lib.pic_compose_seams_workspace(4, 100) >= lib.pic_compose_workspace(4, 100) + 8 * 101


def vrot(lib, form=DENSE, B=1, H=2, dk=128, dv=128, pool=5, idx=(4, 0, 0), shift=(7, -3, 0),
         rot=64, base=10000.0, pairing=0, That=True, ws_bytes=None, S0_out=None, T_out=None):
    i = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    sh = np.ascontiguousarray(np.asarray(shift, dtype=np.int64))
    n = len(i)
    need = lib.pic_rerotate_workspace(n)
    big = 1 << 32  # output buffers far from the pool's
    return lib.pic_validate_rerotate(
        form, B, H, dk, dv, pool, P(0), P(1) if That else None, P(2), n,
        i.ctypes.data_as(ctypes.c_void_p) if n else None,
        sh.ctypes.data_as(ctypes.c_void_p) if n else None, rot, base, pairing,
        ctypes.c_void_p(big), (ctypes.c_void_p(2 * big) if T_out is None else T_out) if That else None,
        ctypes.c_void_p(3 * big) if S0_out is None else S0_out, P(7),
        need if ws_bytes is None else ws_bytes)


def test_validate_rerotate(lib):
    assert vrot(lib) == OK
    assert vrot(lib, form=KDA) == OK
    assert vrot(lib, form=SCALAR, That=False, rot=8, pairing=1) == OK
    assert vrot(lib, form=DIAG, That=False, dk=16, dv=48, rot=16) == OK
    assert vrot(lib, idx=(), shift=()) == OK
    assert lib.pic_last_error().decode() == ""


@pytest.mark.parametrize("kw,code", [
    ({"form": 4}, EUNSUP), ({"pairing": 2}, EUNSUP), ({"base": 0.0}, EUNSUP),
    ({"base": float("inf")}, EUNSUP), ({"base": float("nan")}, EUNSUP),
    ({"rot": 0}, EDIMS), ({"rot": 12}, EDIMS), ({"rot": 136}, EDIMS),
    ({"dk": 16, "dv": 16, "rot": 24}, EDIMS), ({"dk": 8}, EDIMS),
    ({"idx": (4, 5, 0)}, ECHAIN), ({"idx": (-1, 0, 0)}, ECHAIN),
    ({"That": False}, ENULL), ({"form": SCALAR, "That": True}, EUNSUP),
    ({"ws_bytes": 4}, EWS),
    ({"S0_out": ctypes.c_void_p(A * 3 + 16)}, EUNSUP),   # inside the pool's S0
    ({"T_out": ctypes.c_void_p((1 << 32) * 3)}, EUNSUP),  # on top of S0_out
    ({"S0_out": ctypes.c_void_p((1 << 32) * 3 + 4)}, EALIGN),
])
def test_validate_rerotate_rejects(lib, kw, code):
    assert vrot(lib, **kw) == code
    assert lib.pic_last_error().decode() != ""


def vconv(lib, dt=BF16, B=2, H=2, dc=64, W=4, N=100, heads=((0, 0, 0), (40, 40, 3)), n_warm=3,
          ws_bytes=None, y=None, x=None):
    hs = np.ascontiguousarray(np.asarray([h[0] for h in heads], dtype=np.int64))
    he = np.ascontiguousarray(np.asarray([h[1] for h in heads], dtype=np.int64))
    hl = np.ascontiguousarray(np.asarray([h[2] for h in heads], dtype=np.int32))
    n = len(heads)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p) if n else None
    need = lib.pic_conv_warmup_workspace(n)
    return lib.pic_validate_conv_warmup(dt, B, H, dc, W, N, P(0), x or P(1), n, n_warm, p(hs),
                                        p(he), p(hl), y or ctypes.c_void_p(1 << 32), P(3),
                                        need if ws_bytes is None else ws_bytes)


def test_validate_conv_warmup(lib):
    assert vconv(lib) == OK
    assert vconv(lib, dt=F32, W=1, n_warm=0, heads=((5, 0, 0),)) == OK
    assert vconv(lib, heads=()) == OK
    assert vconv(lib, heads=((97, 97, 3),)) == OK  # the last head that fits
    assert lib.pic_last_error().decode() == ""


@pytest.mark.parametrize("kw,code", [
    ({"dt": 3}, EUNSUP), ({"W": 0}, EDIMS), ({"W": 17}, EDIMS), ({"dc": 24}, EDIMS),
    ({"n_warm": 65}, EDIMS), ({"n_warm": -1}, EDIMS),
    ({"heads": ((0, 0, 4),)}, EOFF), ({"heads": ((0, 2, 3),)}, EOFF),
    ({"heads": ((0, 101, 1),)}, EOFF), ({"heads": ((98, 98, 3),)}, EOFF),
    ({"heads": ((-1, 0, 0),)}, EOFF), ({"ws_bytes": 4}, EWS),
    ({"y": ctypes.c_void_p(A * 2 + 32)}, EUNSUP), ({"y": ctypes.c_void_p((1 << 32) + 2)}, EALIGN),
])
def test_validate_conv_warmup_rejects(lib, kw, code):
    assert vconv(lib, **kw) == code
    assert lib.pic_last_error().decode() != ""



# --------------------------------------------------------------------------
# split build: the pieces, the workspace, the argument checks (host only)
# --------------------------------------------------------------------------

def test_split_plan_hand_table(lib):
    """Segments of 0, 1, 64, 65, 200 and 1000 tokens cut into up to 4 pieces
    of whole 64-token chunks (expected offsets worked out by hand)."""
    import hybrid_caching_amd as pic
    offs = [0, 0, 1, 65, 130, 330, 1330]
    pieces, seg_pieces = pic.pic_split_plan(offs, 4)
    assert pieces.tolist() == [0,
                               0,                     # empty segment: one empty piece
                               1,                     # 1 token: one piece
                               65,                    # 64 tokens: one piece
                               129, 130,              # 65 tokens = 2 chunks: 64 + 1
                               194, 258, 322, 330,    # 200 tokens = 4 chunks: one each
                               586, 842, 1098, 1330]  # 1000 tokens = 16 chunks: 4 each
    assert seg_pieces.tolist() == [0, 1, 2, 3, 5, 9, 13]


def test_split_plan_one_piece_is_the_segments(lib):
    import hybrid_caching_amd as pic
    offs = [0, 5, 300, 300, 4096]
    pieces, seg_pieces = pic.pic_split_plan(offs, 1)
    assert pieces.tolist() == offs
    assert seg_pieces.tolist() == [0, 1, 2, 3, 4]


def test_split_plan_errors(lib):
    n_p = ctypes.c_int64(0)
    off, off_p = offsets([0, 200, 400])
    seg = np.zeros(3, dtype=np.int64)
    pieces = np.zeros(2, dtype=np.int64)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.pic_split_plan(2, off_p, 400, 0, P(pieces), 2, P(seg), ctypes.byref(n_p)) == EDIMS
    assert lib.pic_split_plan(2, off_p, 401, 2, P(pieces), 2, P(seg), ctypes.byref(n_p)) == EOFF
    assert lib.pic_split_plan(2, off_p, 400, 2, P(pieces), 2, P(seg), ctypes.byref(n_p)) == EWS
    assert n_p.value == 4  # 200 tokens = 4 chunks: 2 pieces per segment


def test_split_workspace_covers_every_plan(lib):
    """The workspace query bounds the pieces of any segmentation of n_tokens."""
    import hybrid_caching_amd as pic
    rng = np.random.default_rng(9)
    for _ in range(50):
        n_seg = int(rng.integers(1, 12))
        lens = rng.integers(0, 700, size=n_seg)
        offs = np.concatenate([[0], np.cumsum(lens)])
        n_split = int(rng.integers(2, 9))
        pieces, _ = pic.pic_split_plan(offs, n_split)
        P = len(pieces) - 1
        for form, t_hat in ((DENSE, True), (SCALAR, False), (DIAG, False)):
            need_lo = P * 1 * 2 * (128 * 128 * (2 if t_hat else 1) + (128 if form == DIAG else 1)) * 4
            ws = lib.pic_segment_build_split_workspace(form, 1, 2, 128, 128, int(offs[-1]), n_seg,
                                                       n_split)
            assert ws >= need_lo
    assert lib.pic_segment_build_split_workspace(DENSE, 1, 2, 128, 128, 100, 1, 0) == 0


def test_split_build_rejects_before_any_device_call(lib):
    off, off_p = offsets([0, 300, 700])
    args = lambda n_split, ws_bytes: (DENSE, BF16, 0, 1, 2, 128, 128, 700, None, P(0), P(1), P(2),
                                      P(3), off_p, 2, n_split, P(4), P(5), P(6), P(7), ws_bytes,
                                      None)
    assert lib.pic_segment_build_split(*args(0, 1 << 30)) == EDIMS
    assert lib.pic_segment_build_split(*args(4, 64)) == EWS
    bad_off, bad_p = offsets([0, 300, 699])
    a = list(args(4, 1 << 30))
    a[13] = bad_p
    assert lib.pic_segment_build_split(*a) == EOFF
