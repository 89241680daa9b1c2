"""The compose that allocates nothing (pic_compose_noalloc, chain tables in
the library's static scratch) against pic_compose on the same inputs, through
the C ABI: two calls in a row, the second smaller (the scratch keeps the first
call's tables), for the dense and the diagonal forms, with the chain pair, and
the size limit of the scratch."""
import numpy as np
import pytest

import oracle
from oracle import DENSE, DIAG
from tests.gpu_helpers import max_rel_units, report, to_dev
from tests.test_gpu_parity import rand_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def _pool(form, seed):
    import hybrid_caching_amd as pic
    import torch
    rng = np.random.default_rng(seed)
    off = [0] + np.cumsum(rng.integers(1, 130, size=24)).tolist()
    k, v, a, b = rand_case(form, 2, 3, 128, 128, off, seed=seed + 1, alpha=(0.99, 1.0),
                           beta=(0.0, 0.1))
    dt = torch.bfloat16
    return pic.pic_segment_build(form, to_dev(k, dt), to_dev(v, dt), to_dev(a),
                                 to_dev(b) if b is not None else None, off)


def _chains(rng, n_req, lo, hi, pool):
    lens = rng.integers(lo, hi, size=n_req)
    off = [0] + np.cumsum(lens).tolist()
    return off, rng.integers(0, pool, size=off[-1]).tolist()


@pytest.mark.parametrize("form", [DENSE, DIAG])
def test_noalloc_matches_compose_twice(form):
    import hybrid_caching_amd as pic
    import torch
    pair = _pool(form, 70 + form)
    T = pair.get("T_hat")
    rng = np.random.default_rng(71 + form)
    S_in = torch.from_numpy(rng.standard_normal((20, 2, 3, 128, 128)).astype(np.float32)).cuda()
    # first call: 20 requests x 20..39 entries; second: 3 requests x 1..5 entries
    for n_req, lo, hi in ((20, 20, 40), (3, 1, 6)):
        off, idx = _chains(rng, n_req, lo, hi, 24)
        sin = S_in[:n_req].contiguous()
        want = pic.pic_compose(form, pair["log_scale"], T, pair["S0"], off, idx, sin,
                               want_pair=True)
        got = pic.pic_compose_noalloc(form, pair["log_scale"], T, pair["S0"], off, idx, sin,
                                      want_pair=True)
        torch.cuda.synchronize()
        for name, g, w in zip(("S_out", "log_scale_out", "T_hat_out"), got, want):
            if w is None:
                assert g is None
                continue
            g, w = g.cpu().numpy(), w.cpu().numpy()
            e = max_rel_units(g, w, unit_ndim=min(2, w.ndim - 1))
            report(f"form {form}, {n_req} requests: {name} err vs pic_compose {e:.3e}, "
                   f"bitwise {np.array_equal(g, w)}")
            assert e <= 1e-6, name
        # and against the oracle on one sampled chain (layer 1, head 2)
        r = n_req - 1
        ids = idx[off[r]:off[r + 1]]
        lam = pair["log_scale"].cpu().numpy()[ids][:, 1:2, 2:3]
        S0 = pair["S0"].cpu().numpy()[ids][:, 1:2, 2:3]
        Th = T.cpu().numpy()[ids][:, 1:2, 2:3] if T is not None else None
        ref = oracle.compose(form, lam, Th, S0, [0, len(ids)], list(range(len(ids))),
                             S_in[r:r + 1, 1:2, 2:3].cpu().numpy())
        e = max_rel_units(got[0][r, 1, 2].cpu().numpy(), ref[0, 0, 0])
        report(f"form {form}, {n_req} requests: chain {r} err vs oracle {e:.3e}")
        assert e <= 1e-4


def test_noalloc_rejects_tables_beyond_the_scratch():
    import hybrid_caching_amd as pic
    from hybrid_caching_amd import _lib
    pair = _pool(DENSE, 90)
    n = 300_000  # 1.2 MB of int32 pool indices > 1 MiB
    with pytest.raises(_lib.PicError) as ei:
        pic.pic_compose_noalloc(DENSE, pair["log_scale"], pair["T_hat"], pair["S0"], [0, n],
                                [0] * n)
    assert ei.value.code == -5 and "scratch" in str(ei.value)
