"""The five reference workloads at full size, in the launch configuration the
benchmark times (same entry points, same shapes, same streams).

The three small workloads are compared with the oracle on every element.
For the two ~1 GB float16 workloads the oracle runs on a seeded sample of
rows (rows are independent, so a sampled row's reference is exact), and two
properties are checked on every element: S equals numpy's own float32 sum
rounded to float16, and every output is finite."""
import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
from group_normalization_amd import workloads
from parity import assert_bitwise, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def sample_rows(n_rows, k, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(n_rows, size=min(k, n_rows), replace=False)
    return np.unique(np.concatenate([rows, [0, n_rows - 1]]))


def test_ssln_f32_64x768():
    w = W["ssln_f32_64x768"]
    x = workloads.generate(w)
    eps = w.attrs["epsilon"]
    out = gn.skip_rms_norm(to_dev(x["input"]), to_dev(x["skip"]), to_dev(x["gamma"]), to_dev(x["bias"]),
                           eps, want_inv_std_var=True, want_sum=True)
    ref = oracle.skip_rms_norm(x["input"], x["skip"], x["gamma"], x["bias"], eps,
                               want_inv_std_var=True, want_sum=True)
    assert_close(to_host(out.output), ref[0], "output")
    assert_close(to_host(out.inv_std_var), ref[2], "inv_std_var")
    assert_bitwise(to_host(out.input_skip_bias_sum), ref[3], "S")


def test_ssln_f16_16x2048x4096_sampled():
    w = W["ssln_f16_16x2048x4096"]
    x = workloads.generate(w)
    eps = w.attrs["epsilon"]
    out = gn.skip_rms_norm(to_dev(x["input"]), to_dev(x["skip"]), to_dev(x["gamma"]), None, eps,
                           want_sum=True)
    assert gn.last_route() == "ssln.wave2.vec16"
    y = to_host(out.output).reshape(-1, 4096)
    s = to_host(out.input_skip_bias_sum).reshape(-1, 4096)
    inp, skp = x["input"].reshape(-1, 4096), x["skip"].reshape(-1, 4096)
    rows = sample_rows(inp.shape[0], 512, seed=20)
    ref = oracle.skip_rms_norm(inp[rows], skp[rows], x["gamma"], None, eps, want_sum=True)
    assert_close(y[rows], ref[0], "output (sampled rows)")
    assert_bitwise(s[rows], ref[3], "S (sampled rows)")
    for lo in range(0, inp.shape[0], 4096):  # every element, in chunks
        hi = lo + 4096
        want = (inp[lo:hi].astype(np.float32) + skp[lo:hi].astype(np.float32)).astype(np.float16)
        assert_bitwise(s[lo:hi], want, f"S rows {lo}:{hi}")
    assert np.isfinite(y).all()


def test_gated_f16_8x4096x4096_c128_sampled():
    w = W["gated_f16_8x4096x4096_c128"]
    x = workloads.generate(w)
    y = to_host(gn.gated_rms_norm(to_dev(x["X"]), to_dev(x["scale"]), to_dev(x["gate"]),
                                  w.attrs["epsilon"]))
    assert gn.last_route() == "gated.segment.vec16"
    y = y.reshape(-1, 128)
    X, G = x["X"].reshape(-1, 128), x["gate"].reshape(-1, 128)
    rows = sample_rows(X.shape[0], 4096, seed=21)
    ref = oracle.gated_rms_norm(X[rows], x["scale"], G[rows], w.attrs["epsilon"])
    assert_close(y[rows], ref, "Y (sampled rows)")
    assert np.isfinite(y).all()


@pytest.mark.parametrize("name", ["sgn_f16_nhwc_2x64x64x320", "sgn_f32_nchw_4x1280x32x32"])
def test_sgn_full(name):
    w = W[name]
    x = workloads.generate(w)
    a = w.attrs
    want_sum = "S" in w.outputs
    out = gn.skip_group_norm(to_dev(x["X"]), to_dev(x["gamma"]), to_dev(x["beta"]), to_dev(x["skip"]),
                             to_dev(x.get("bias")), groups=a["groups"], activation=a["activation"],
                             epsilon=a["epsilon"], channels_last=a["channels_last"],
                             want_sum=want_sum)
    assert gn.last_route() == ("sgn.cluster.nhwc.vec16" if a["channels_last"] else "sgn.cluster.nchw.vec16")
    ref_y, ref_s = oracle.skip_group_norm(x["X"], x["gamma"], x["beta"], x["skip"], x.get("bias"),
                                          groups=a["groups"], activation=a["activation"],
                                          epsilon=a["epsilon"], channels_last=a["channels_last"],
                                          want_sum=True)
    assert_close(to_host(out.Y), ref_y, "Y")
    if want_sum:
        assert_bitwise(to_host(out.S), ref_s, "S")
