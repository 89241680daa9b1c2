"""The fp16-operand calls' overflow report, through the C ABI: a build or
prefill at fp16 operand precision whose inputs leave fp16's range (|v| above
its largest finite value, outside the PIC_PREC_FP16 preconditions) stores
values that are not finite and sets the device flag, which
pic_nonfinite_check reports once and clears; in-range inputs, and the fp32
path on the same out-of-range inputs, leave it clear.
"""
import numpy as np
import pytest

import synth
from oracle import DENSE
from tests.gpu_helpers import to_dev
from tests.test_gpu_parity import RAGGED, rand_case

pytestmark = pytest.mark.gpu

NONFINITE = -9


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_caching_amd as pic
    pic.load()


def _clear():
    import hybrid_caching_amd as pic
    try:
        pic.pic_nonfinite_check()
    except pic.PicError:
        pass


def _case(v_scale):
    k, v, a, b = rand_case(DENSE, 2, 3, 64, 64, RAGGED, seed=4242)
    v = synth.bf16_round((v * v_scale).astype(np.float32))
    q = synth.bf16_round(np.random.default_rng(4243).standard_normal(k.shape).astype(np.float32))
    return q, k, v, a, b


def _build(q, k, v, a, b, precision):
    import hybrid_caching_amd as pic
    import torch
    bf = torch.bfloat16
    return pic.pic_segment_build(DENSE, to_dev(k, bf), to_dev(v, bf), to_dev(a), to_dev(b), RAGGED,
                                 precision=precision)


def test_in_range_build_and_prefill_leave_the_flag_clear():
    import hybrid_caching_amd as pic
    import torch
    _clear()
    q, k, v, a, b = _case(1.0)
    out = _build(q, k, v, a, b, pic.PREC_FP16)
    bf = torch.bfloat16
    pf = pic.pic_segment_prefill(to_dev(q, bf), to_dev(k, bf), to_dev(v, bf), to_dev(a),
                                 to_dev(b), RAGGED, check_finite=True)
    pic.pic_nonfinite_check()
    assert torch.isfinite(out["S0"]).all() and torch.isfinite(pf["O"].float()).all()


def test_fp16_build_overflow_is_reported_once():
    import hybrid_caching_amd as pic
    import torch
    _clear()
    q, k, v, a, b = _case(1e6)  # |v| far above fp16's largest finite value
    out = _build(q, k, v, a, b, pic.PREC_FP16)
    torch.cuda.synchronize()
    assert not torch.isfinite(out["S0"]).all()
    with pytest.raises(pic.PicError) as err:
        pic.pic_nonfinite_check()
    assert err.value.code == NONFINITE
    pic.pic_nonfinite_check()  # cleared by the check that reported it
    # the same inputs on the fp32 path: finite results, no report
    out32 = _build(q, k, v, a, b, pic.PREC_FP32)
    torch.cuda.synchronize()
    assert torch.isfinite(out32["S0"]).all()
    pic.pic_nonfinite_check()


def test_fp16_prefill_overflow_raises_with_check_finite():
    import hybrid_caching_amd as pic
    import torch
    _clear()
    q, k, v, a, b = _case(1e6)
    bf = torch.bfloat16
    with pytest.raises(pic.PicError) as err:
        pic.pic_segment_prefill(to_dev(q, bf), to_dev(k, bf), to_dev(v, bf), to_dev(a), to_dev(b),
                                RAGGED, check_finite=True)
    assert err.value.code == NONFINITE
    pic.pic_nonfinite_check()
