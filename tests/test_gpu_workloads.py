"""The five reference workloads at full size, in the launch configuration the
benchmark times (same entry points, same shapes, same streams).

Every output element of every workload is compared with the oracle.  For the
two ~1 GB float16 workloads the single-threaded oracle runs over chunks of
whole rows in a thread pool (rows are independent; each chunk is one plain
serial oracle call, and ctypes releases the GIL while it runs), and each
chunk is compared with the GPU's rows as soon as it is done.  As a second
opinion, the SkipSimplifiedLayerNormalization sum S is also checked against
numpy's own float32 sum rounded to float16."""
import concurrent.futures
import os

import numpy as np
import pytest

import group_normalization_amd as gn
import oracle
import workloads
from parity import assert_bitwise, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
CHUNK_ROWS = 2048


def over_row_chunks(n_rows, check_chunk):
    """Run check_chunk(lo, hi) over [0, n_rows) in chunks of CHUNK_ROWS rows on
    a thread pool; re-raise the first failure with its row range."""
    workers = max(1, min(16, os.cpu_count() or 1))
    bounds = [(lo, min(n_rows, lo + CHUNK_ROWS)) for lo in range(0, n_rows, CHUNK_ROWS)]
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futures = {ex.submit(check_chunk, lo, hi): (lo, hi) for lo, hi in bounds}
        for f in concurrent.futures.as_completed(futures):
            lo, hi = futures[f]
            try:
                f.result()
            except AssertionError as e:
                raise AssertionError(f"rows {lo}:{hi}: {e}") from None
    return len(bounds)


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


def test_ssln_f16_16x2048x4096_every_row():
    w = W["ssln_f16_16x2048x4096"]
    x = workloads.generate(w)
    eps = w.attrs["epsilon"]
    out = gn.skip_rms_norm(to_dev(x["input"]), to_dev(x["skip"]), to_dev(x["gamma"]), None, eps,
                           want_sum=True)
    assert gn.last_route() == "ssln.wave2.vec16"
    y = to_host(out.output).reshape(-1, 4096)
    s = to_host(out.input_skip_bias_sum).reshape(-1, 4096)
    del out
    inp, skp = x["input"].reshape(-1, 4096), x["skip"].reshape(-1, 4096)
    gamma = x["gamma"]

    def check_chunk(lo, hi):
        ref = oracle.skip_rms_norm(inp[lo:hi], skp[lo:hi], gamma, None, eps, want_sum=True)
        assert_close(y[lo:hi], ref[0], "output")
        assert_bitwise(s[lo:hi], ref[3], "S")
        # Second opinion on S: numpy's float32 sum, rounded once to float16.
        want = (inp[lo:hi].astype(np.float32) + skp[lo:hi].astype(np.float32)).astype(np.float16)
        assert_bitwise(s[lo:hi], want, "S (numpy)")

    assert over_row_chunks(inp.shape[0], check_chunk) == 16


def test_gated_f16_8x4096x4096_c128_every_row():
    w = W["gated_f16_8x4096x4096_c128"]
    x = workloads.generate(w)
    eps = w.attrs["epsilon"]
    y = to_host(gn.gated_rms_norm(to_dev(x["X"]), to_dev(x["scale"]), to_dev(x["gate"]), eps))
    assert gn.last_route() == "gated.segment.vec16"
    y = y.reshape(-1, 128)
    X, G = x["X"].reshape(-1, 128), x["gate"].reshape(-1, 128)
    scale = x["scale"]

    def check_chunk(lo, hi):
        assert_close(y[lo:hi], oracle.gated_rms_norm(X[lo:hi], scale, G[lo:hi], eps), "Y")

    assert over_row_chunks(X.shape[0], check_chunk) == 512


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
