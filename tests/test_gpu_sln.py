"""Skip layer normalization with the row mean removed (the non-simplified
form of SkipSimplifiedLayerNormalization): HIP path through the C ABI
against the oracle, element by element, on every route."""
import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
import workloads
from parity import assert_bitwise, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

F32, F16 = np.float32, np.float16


def run_both(x, eps, route="auto", want=("mean", "inv", "sum")):
    ref = oracle.skip_layer_norm(x["input"], x["skip"], x["gamma"], x.get("beta"), x.get("bias"), eps,
                                 want_mean=True, want_inv_std_var=True, want_sum=True)
    with gn.force_route(route):
        out = gn.skip_layer_norm(to_dev(x["input"]), to_dev(x["skip"]), to_dev(x["gamma"]),
                                 to_dev(x.get("beta")), to_dev(x.get("bias")), eps,
                                 want_mean="mean" in want, want_inv_std_var="inv" in want,
                                 want_sum="sum" in want)
        used = gn.last_route()
    torch.cuda.synchronize()
    return ref, out, used


def check(ref, out, want=("mean", "inv", "sum")):
    y_ref, mean_ref, inv_ref, s_ref = ref
    assert_close(to_host(out.output), y_ref, "output")
    if "sum" in want:
        assert_bitwise(to_host(out.input_skip_bias_sum), s_ref, "input_skip_bias_sum")
    if "inv" in want:
        assert_close(to_host(out.inv_std_var), inv_ref, "inv_std_var")
    if "mean" in want:
        assert_close(to_host(out.mean), mean_ref, "mean")


SHAPES = [
    # (shape, dtype, beta, bias): every route of the row kernels
    ((64, 768), F32, True, True),       # one wave per row
    ((13, 768), F16, False, False),
    ((3, 5, 4096), F16, True, False),   # two waves per row, odd row count
    ((7, 8192), F16, True, True),       # four waves per row
    ((5, 8192), F32, False, True),      # eight waves per row
    ((3, 20480), F16, True, False),     # sixteen waves per row, ragged
    ((2, 16384), F32, True, True),      # float32, sixteen waves per row
    ((9, 1000), F16, True, False),      # ragged lanes
    ((6, 33), F32, True, False),        # scalars
    ((4, 1), F16, True, True),          # one element: variance 0
    ((3, 4100), F16, True, False),      # 8-byte vectors
    ((3, 4098), F16, False, True),      # 4-byte vectors
    ((2, 4097), F16, True, False),      # odd width: phased route
    ((2, 40000), F16, True, True),      # sixteen waves, 5 vectors per lane
    ((2, 65544), F16, True, True),      # block route (three passes), 16-byte vectors
    ((2, 40000), F32, False, True),     # float32 block route
    ((3, 20002), F32, True, False),     # rows off the 16-byte grid: phased route
    ((2, 8193), F16, False, True),      # odd: phased route
    ((2, 16385), F16, False, True),     # odd: phased route, sixteen waves
    ((2, 32769), F16, True, True),      # block route, scalars
    ((2, 100000), F16, True, True),     # wide route: 8 vectors per lane in VGPRs, 5 in LDS
    ((3, 139264), F16, False, False),   # wide route at its widest
    ((2, 69632), F32, True, False),     # float32 wide route at its widest
    ((2, 40004), F32, False, True),     # float32 wide route, ragged
    ((2, 139272), F16, True, False),    # past the wide route: block route
    ((1000, 128), F16, True, True),     # lane groups: 16 lanes per row
    ((64, 6), F32, True, False),        # lane groups of 4
    ((31, 7), F16, True, True),         # scalars in lane groups of 8
]


@pytest.mark.parametrize("route", ["auto", "scalar", "block"])
@pytest.mark.parametrize("shape,dt,beta,bias", SHAPES,
                         ids=[f"{s}-{np.dtype(d).name}{'-beta' if be else ''}{'-bias' if b else ''}"
                              for s, d, be, b in SHAPES])
def test_matches_oracle(shape, dt, beta, bias, route):
    w = workloads.sln("t", shape, dt, beta=beta, bias=bias, epsilon=1e-5)
    x = workloads.generate(w, seed=sum(shape) + 1)
    ref, out, used = run_both(x, 1e-5, route)
    check(ref, out)
    if route == "block":
        assert used == "ssln.block"
    elif route == "auto" and shape[-1] * np.dtype(dt).itemsize > 131072:
        # Wider than 1024 lanes x 8 x 16 bytes: rows of 16-byte vectors up to
        # 17 per lane (9 of them in LDS) take the wide route, others the block route.
        width16 = shape[-1] * np.dtype(dt).itemsize % 16 == 0
        if width16 and shape[-1] * np.dtype(dt).itemsize <= 1024 * 17 * 16:
            assert used == "ssln.wide.vec16"
        else:
            assert used.startswith("ssln.block")


NON_FINITE_SHAPES = [
    # (shape, dtype): one shape for each row route
    ((64, 768), F32),       # one wave per row
    ((7, 8192), F16),       # four waves per row
    ((3, 4100), F16),       # 8-byte vectors
    ((3, 4097), F16),       # phased route
    ((1000, 128), F16),     # flat route, lane groups of 16
    ((31, 7), F16),         # flat route, scalars
    ((3, 100000), F16),     # wide route
    ((3, 65544), F16),      # block route
    ((3, 33), F32),         # short odd float32 rows
]


@pytest.mark.parametrize("route", ["auto", "block"])
@pytest.mark.parametrize("shape,dt", NON_FINITE_SHAPES, ids=[f"{s}-{np.dtype(d).name}" for s, d in NON_FINITE_SHAPES])
def test_non_finite_rows(shape, dt, route):
    """Rows whose sum overflows to +inf at their first element (the element
    the kernels take their sums about), +inf further in, and a NaN first
    element: the mean is the row's sum over its count (+inf, or NaN), the
    variance NaN, so inv_std_var and every output of the row are NaN, as in
    the oracle; S keeps the infinities bit for bit and the other rows are
    untouched."""
    w = workloads.sln("t", shape, dt, beta=True, bias=True, epsilon=1e-5)
    x = workloads.generate(w, seed=sum(shape) + 3)
    inp, skp = x["input"].copy(), x["skip"].copy()
    hidden = shape[-1]
    a, k = inp.reshape(-1, hidden), skp.reshape(-1, hidden)
    big = 65504.0 if dt == F16 else 3e38
    a[0, 0] = k[0, 0] = big                      # S[0] = +inf
    a[1, hidden // 2] = k[1, hidden // 2] = big  # +inf inside the row
    a[2, 0] = np.nan                             # S[0] = NaN
    x = dict(x, input=inp, skip=skp)
    ref, out, used = run_both(x, 1e-5, route)
    check(ref, out)
    mean = to_host(out.mean).reshape(-1)
    assert mean[0] == np.inf and mean[1] == np.inf and np.isnan(mean[2]), (used, mean[:3])
    y = to_host(out.output).reshape(-1, hidden)
    assert np.isnan(y[:3]).all() and np.isfinite(y[3:]).all(), used


@pytest.mark.parametrize("want", [(), ("sum",), ("mean",), ("inv",), ("mean", "inv", "sum")])
@pytest.mark.parametrize("dt,hidden", [(F32, 2048), (F16, 4096), (F16, 16384), (F32, 50000)])
def test_optional_outputs_do_not_change_output(dt, hidden, want):
    w = workloads.sln("t", (21, hidden), dt, beta=True, bias=True, epsilon=1e-5)
    x = workloads.generate(w, seed=7)
    ref, out, _ = run_both(x, 1e-5, want=want)
    check(ref, out, want)
    _, base, _ = run_both(x, 1e-5, want=())
    assert_bitwise(to_host(out.output), to_host(base.output), "output with/without optional outputs")


@pytest.mark.parametrize("route", ["auto", "block"])
def test_constant_rows_give_beta(route):
    rows, hidden = 5, 640
    x = {"input": np.full((rows, hidden), 1.5, F32), "skip": np.full((rows, hidden), -0.25, F32),
         "gamma": np.linspace(-2, 2, hidden).astype(F32), "beta": np.linspace(3, -1, hidden).astype(F32)}
    ref, out, _ = run_both(x, 1e-5, route)
    check(ref, out)
    assert np.array_equal(to_host(out.output), np.broadcast_to(x["beta"], (rows, hidden)))
    assert np.all(to_host(out.mean) == np.float32(1.25))


def test_large_mean_is_removed():
    """Rows far from zero (mean 1000, spread 1): the statistics come from the
    S held in registers in two passes, so the variance keeps its accuracy."""
    rng = np.random.default_rng(5)
    rows, hidden = 8, 4096
    x = {"input": (1000 + rng.standard_normal((rows, hidden))).astype(F32),
         "skip": (0.5 * rng.standard_normal((rows, hidden))).astype(F32),
         "gamma": np.ones(hidden, F32)}
    ref, out, _ = run_both(x, 1e-5)
    check(ref, out)


def test_deterministic():
    w = workloads.sln("t", (64, 4096), F16, beta=True, bias=True, epsilon=1e-5)
    x = workloads.generate(w, seed=9)
    a = run_both(x, 1e-5)[1]
    b = run_both(x, 1e-5)[1]
    for f in ("output", "mean", "inv_std_var", "input_skip_bias_sum"):
        assert_bitwise(to_host(getattr(a, f)), to_host(getattr(b, f)), f)


def test_workload_sampled_rows():
    """The 16x2048x4096 float16 workload at full size; sampled rows checked
    against the oracle, S bit for bit."""
    w = workloads.EXTRA_WORKLOADS["sln_f16_16x2048x4096"]
    x = workloads.generate(w)
    d = {k: to_dev(v) for k, v in x.items()}
    out = gn.skip_layer_norm(d["input"], d["skip"], d["gamma"], d["beta"], None, 1e-5, want_sum=True,
                             want_mean=True, want_inv_std_var=True)
    assert gn.last_route() == "ssln.wave2.vec16"
    torch.cuda.synchronize()
    hidden = 4096
    inp, skp = x["input"].reshape(-1, hidden), x["skip"].reshape(-1, hidden)
    rows = np.array([0, 1, 2047, 2048, 16000, inp.shape[0] - 1])
    ref = oracle.skip_layer_norm(inp[rows], skp[rows], x["gamma"], x["beta"], None, 1e-5, want_mean=True,
                                 want_inv_std_var=True, want_sum=True)
    y = to_host(out.output).reshape(-1, hidden)[rows]
    assert_close(y, ref[0], "output")
    assert_close(to_host(out.mean).reshape(-1, 1)[rows], ref[1], "mean")
    assert_close(to_host(out.inv_std_var).reshape(-1, 1)[rows], ref[2], "inv_std_var")
    assert_bitwise(to_host(out.input_skip_bias_sum).reshape(-1, hidden)[rows], ref[3], "S")
