import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def rel_fro(x, ref):
    """Relative Frobenius error ||x - ref|| / ||ref|| (0/0 counts as 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm((x - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if np.isnan(num) or np.isnan(den):
        return np.inf
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return num / den


def rel_fro_units(x, ref, unit_ndim=2):
    """Maximum over units of the relative Frobenius error, where a unit is the
    trailing ``unit_ndim`` axes (one state or one operator)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lead = x.shape[: x.ndim - unit_ndim]
    xs = x.reshape((-1,) + x.shape[x.ndim - unit_ndim:])
    rs = ref.reshape((-1,) + ref.shape[ref.ndim - unit_ndim:])
    worst = 0.0
    for a, b in zip(xs, rs):
        e = rel_fro(a, b)
        if not e <= worst:  # NaN counts as the worst error
            worst = e if not np.isnan(e) else np.inf
    return worst


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    return oracle.load()
