"""The parity bound itself (CPU): half-ulp arithmetic and the bound's independence
from the output under test."""
import numpy as np

from parity_util import check_out, half_ulp_bf16, tolerance, workload
from workloads import gen


def test_half_ulp_matches_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-10, 10, 200000))).astype(np.float32)
    r = gen.round_bf16_np(x).astype(np.float64)
    assert np.all(np.abs(r - x.astype(np.float64)) <= half_ulp_bf16(x.astype(np.float64)))
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0**-8
    assert half_ulp_bf16(np.array([0.75]))[0] == 2.0**-9


def test_bound_rejects_large_errors():
    w = workload(dtype="bf16")
    ref = np.random.default_rng(1).standard_normal((50, 8)) * 0.1
    t = tolerance(w, ref)
    assert np.all(t < 0.01)
    bad = ref.copy()
    bad[3, 2] = 1e6
    try:
        check_out(w, bad, ref)
    except AssertionError:
        pass
    else:
        raise AssertionError("bound accepted a wild output")
    # the correctly rounded reference always passes
    check_out(w, gen.round_bf16_np(ref.astype(np.float32)).astype(np.float64), ref)
