"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the oracle on the same values, compare."""
import os

import numpy as np

import oracle
from tests.conftest import rel_fro

# Contract tolerances (relative Frobenius per unit): fp32 state with fp32
# inputs, and with bf16 q/k/v inputs.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(x, dtype=None):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def qkv_dtype(bf16: bool):
    import torch
    return torch.bfloat16 if bf16 else torch.float32


def max_rel_units(got, ref, unit_ndim=2):
    """Max over units of the relative Frobenius error; a unit = trailing dims.
    Magnitudes below the smallest fp32 normal count as zero on both sides."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tiny = np.finfo(np.float32).tiny
    got = np.where(np.abs(got) < tiny, 0.0, got)
    ref = np.where(np.abs(ref) < tiny, 0.0, ref)
    g = got.reshape((-1,) + got.shape[got.ndim - unit_ndim:])
    r = ref.reshape((-1,) + ref.shape[ref.ndim - unit_ndim:])
    worst = 0.0
    for a, b in zip(g, r):
        e = rel_fro(a, b)
        if not e <= worst:  # NaN counts as the worst error
            worst = e if not np.isnan(e) else np.inf
    return worst


def lam_err(got, ref):
    """max |dlam| / max(1, |lam|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def build_both(form, k, v, alpha, beta, offsets, bf16, q=None, precision=0):
    """Run the HIP build and the oracle on the same (numpy, fp32-exact) inputs."""
    import hybrid_caching_amd as pic
    import torch
    dt = qkv_dtype(bf16)
    out = pic.pic_segment_build(form, to_dev(k, dt), to_dev(v, dt), to_dev(alpha),
                                to_dev(beta), offsets, q=None if q is None else to_dev(q, dt),
                                precision=precision)
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in out.items()}
    ref = oracle.build(form, k, v, alpha, beta, offsets)
    return gpu, ref


def report(line: str):
    """Print a measured error and, if PIC_PARITY_LOG names a file, append it there."""
    print(line)
    path = os.environ.get("PIC_PARITY_LOG")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a", encoding="utf-8") as f:
            f.write(f"{test}: {line}\n")


def assert_pair_close(gpu, ref, form, tol):
    e_s = max_rel_units(gpu["S0"], ref["S"])
    e_l = lam_err(gpu["log_scale"], ref["lam"])
    msg = f"S0 err {e_s:.3e}, lambda err {e_l:.3e}"
    e_t = 0.0
    if form in (oracle.DENSE, oracle.KDA):
        e_t = max_rel_units(gpu["T_hat"], ref["That"])
        msg += f", That err {e_t:.3e}"
    report(msg)
    assert e_t <= tol, msg
    assert e_s <= tol, msg
    assert e_l <= 1e-4, msg
    return msg
