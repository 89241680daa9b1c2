"""Plan tables too large for the kernel arguments reach the device either
straight from host memory (the default: the call waits for its stream and the
library holds no memory afterwards) or through the opt-in pinned pool.  Both
ways give the same results, the default holds no memory, and a release
returns the library to holding none."""
import numpy as np
import pytest

from oracle import DENSE
from tests.gpu_helpers import to_dev
from tests.test_gpu_parity import rand_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def _large_calls():
    """A build of 40 segments and a compose of 20 requests x 70 entries: both
    plans exceed what travels in the kernel arguments."""
    import hybrid_caching_amd as pic
    import torch
    rng = np.random.default_rng(44)
    lens = rng.integers(0, 150, size=40)
    off = [0] + np.cumsum(lens).tolist()
    k, v, a, b = rand_case(DENSE, 1, 2, 64, 64, off, seed=45)
    dt = torch.bfloat16
    pair = pic.pic_segment_build(DENSE, to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(b), off)
    c_off = [0] + np.cumsum(rng.integers(50, 90, size=20)).tolist()
    idx = rng.integers(0, 40, size=c_off[-1]).tolist()
    S = pic.pic_compose(DENSE, pair["log_scale"], pair["T_hat"], pair["S0"], c_off, idx)
    torch.cuda.synchronize()
    return {key: t.cpu().numpy() for key, t in pair.items()}, S.cpu().numpy()


def test_default_holds_no_memory_and_pool_is_released():
    import hybrid_caching_amd as pic
    pic.pic_staging_release()
    assert pic.pic_staging_bytes() == 0
    pair0, S0 = _large_calls()
    assert pic.pic_staging_bytes() == 0
    pic.pic_staging_reserve()
    assert pic.pic_staging_bytes() == 64 * 64 * 1024
    pic.pic_staging_reserve()  # a second reserve on the device does nothing
    assert pic.pic_staging_bytes() == 64 * 64 * 1024
    for _ in range(3):  # more calls than one slot's reuse
        pair1, S1 = _large_calls()
        for key in pair0:
            assert np.array_equal(pair0[key], pair1[key]), key
        assert np.array_equal(S0, S1)
    pic.pic_staging_release()
    assert pic.pic_staging_bytes() == 0
    pair2, S2 = _large_calls()
    assert np.array_equal(S0, S2)
