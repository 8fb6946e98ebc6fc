"""The usage examples' shapes from the operator pages (their data are
placeholders there, so the data here are seeded): SkipGroupNorm with X
(2, 3, 2, 8) in the default NHWC layout, a broadcast skip (2, 8), groups 2,
no activation (SGN page, usage example); SkipSimplifiedLayerNormalization
with input and skip (2, 4) and gamma (4) and the default epsilon (SSLN page,
usage example).  The GatedRMSNorm example (X, gate (3, 4), scale (1)) is
in test_gpu_gated.py.  Every route, both data types."""
import numpy as np
import pytest

import group_normalization_amd as gn
import oracle
import workloads
from parity import assert_bitwise, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

F32, F16 = np.float32, np.float16


@pytest.mark.parametrize("route", ["auto", "split", "scalar", "block"])
@pytest.mark.parametrize("dt", [F32, F16])
def test_sgn_page_example(dt, route):
    w = workloads.sgn("t", 2, 8, 3, 2, dt, F32, channels_last=True, broadcast_skip=True, bias=False,
                      groups=2, activation=0, epsilon=1e-5)
    x = workloads.generate(w, seed=21)
    assert x["X"].shape == (2, 3, 2, 8) and x["skip"].shape == (2, 8)
    ref_y, ref_s = oracle.skip_group_norm(x["X"], x["gamma"], x["beta"], x["skip"], None, groups=2,
                                          activation=0, want_sum=True)
    with gn.force_route(route):
        out = gn.skip_group_norm(to_dev(x["X"]), to_dev(x["gamma"]), to_dev(x["beta"]), to_dev(x["skip"]),
                                 groups=2, activation=0, want_sum=True)
    assert_close(to_host(out.Y), ref_y, "Y")
    assert_bitwise(to_host(out.S), ref_s, "S")


@pytest.mark.parametrize("route", ["auto", "scalar", "block"])
@pytest.mark.parametrize("dt", [F32, F16])
def test_ssln_page_example(dt, route):
    w = workloads.ssln("t", (2, 4), dt, bias=False, epsilon=gn.SSLN_EPSILON)
    x = workloads.generate(w, seed=22)
    ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], None, gn.SSLN_EPSILON,
                               want_mean=True, want_inv_std_var=True, want_sum=True)
    with gn.force_route(route):
        out = gn.skip_rms_norm(to_dev(x["input"]), to_dev(x["skip"]), to_dev(x["gamma"]),
                               want_mean=True, want_inv_std_var=True, want_sum=True)
    assert_close(to_host(out.output), ref[0], "output")
    assert np.all(to_host(out.mean) == 0)
    assert_close(to_host(out.inv_std_var), ref[2], "inv_std_var")
    assert_bitwise(to_host(out.input_skip_bias_sum), ref[3], "S")
