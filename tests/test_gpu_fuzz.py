"""Seeded random parity: shapes, dtypes, optional inputs and outputs and
unaligned base addresses drawn at random (fixed seeds, so every run checks
the same cases) for every operator, each compared with the oracle element by
element (S bitwise).  The draws cover the length buckets that select the
different routes and access widths, so that combinations the hand-written
cases miss are still exercised."""
import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
from parity import assert_bitwise, assert_bitwise_nan, assert_close, to_host

pytestmark = pytest.mark.gpu

F32, F16 = np.float32, np.float16
MAX_ELEMS = 1 << 21
N_CASES = 64


def dev(a, offset=0):
    """a on the GPU, starting `offset` elements into a fresh buffer (a
    contiguous view whose base address is shifted)."""
    if a is None:
        return None
    flat = torch.empty(a.size + offset, dtype=torch.float16 if a.dtype == F16 else torch.float32,
                       device="cuda")
    view = flat[offset:]
    view.copy_(torch.from_numpy(np.ascontiguousarray(a).ravel()))
    return view.view(a.shape)


def draw_length(rng, buckets):
    los, his, ps = zip(*buckets)
    i = rng.choice(len(buckets), p=np.array(ps) / sum(ps))
    return int(rng.integers(los[i], his[i] + 1))


def normal(rng, shape, dtype, scale=1.0):
    return (scale * rng.standard_normal(shape)).astype(dtype)


def uniform(rng, shape, dtype):
    return rng.uniform(0.5, 1.5, shape).astype(dtype)


def plant(rng, a, b, dt, k):
    """k non-finite values at random positions of a: +inf, -inf, NaN, or a
    pair of equal large finite values in a and b at the same position (their
    sum overflows dt).  b may be None (no pair then)."""
    big = 65504.0 if dt == F16 else 3e38
    fa, fb = a.reshape(-1), None if b is None else b.reshape(-1)
    for i in rng.choice(fa.size, size=min(k, fa.size), replace=False):
        kind = int(rng.integers(0, 4 if fb is not None else 3))
        if kind == 3:
            fa[i] = fb[i] = big
        else:
            fa[i] = (np.inf, -np.inf, np.nan)[kind]


N_NON_FINITE = 24


@pytest.mark.parametrize("case", range(N_CASES))
@pytest.mark.parametrize("center", [False, True], ids=["ssln", "sln"])
def test_row_norms(center, case):
    row_norms(center, np.random.default_rng(1000 + case + (500 if center else 0)), False)


@pytest.mark.parametrize("case", range(N_NON_FINITE))
@pytest.mark.parametrize("center", [False, True], ids=["ssln", "sln"])
def test_row_norms_non_finite(center, case):
    """As test_row_norms, with a few infinities, NaNs and overflowing sums at
    random positions: every output (NaN positions and infinities exactly)
    equals the oracle's."""
    row_norms(center, np.random.default_rng(4000 + case + (500 if center else 0)), True)


def row_norms(center, rng, non_finite):
    dt = F16 if rng.random() < 0.6 else F32
    hidden = draw_length(rng, [(1, 64, 4), (65, 2048, 3), (2049, 12000, 2), (12001, 70000, 1)])
    rows = int(rng.integers(1, max(2, min(300, MAX_ELEMS // hidden)) + 1))
    shape = (rows, hidden) if rng.random() < 0.7 else (1, rows, hidden)
    x, k = normal(rng, shape, dt), normal(rng, shape, dt)
    gamma = uniform(rng, hidden, dt)
    bias = normal(rng, hidden, dt, 0.1) if rng.random() < 0.5 else None
    beta = normal(rng, hidden, dt, 0.1) if center and rng.random() < 0.6 else None
    if non_finite:
        plant(rng, x, k, dt, int(rng.integers(1, 6)))
    off = int(rng.choice([0, 0, 0, 1, 2, 4]))
    eps = float(rng.choice([1e-6, 1e-5]))
    want = {w: bool(rng.random() < 0.5) for w in ("mean", "inv", "sum")}
    if center:
        ref = oracle.skip_layer_norm(x.reshape(-1, hidden), k.reshape(-1, hidden), gamma, beta, bias, eps,
                                     want_mean=True, want_inv_std_var=True, want_sum=True)
        out = gn.skip_layer_norm(dev(x, off), dev(k, off), dev(gamma), dev(beta), dev(bias), eps,
                                 want_mean=want["mean"], want_inv_std_var=want["inv"], want_sum=want["sum"])
    else:
        ref = oracle.skip_rms_norm(x.reshape(-1, hidden), k.reshape(-1, hidden), gamma, bias, eps,
                                   want_mean=True, want_inv_std_var=True, want_sum=True)
        out = gn.skip_rms_norm(dev(x, off), dev(k, off), dev(gamma), dev(bias), eps,
                               want_mean=want["mean"], want_inv_std_var=want["inv"], want_sum=want["sum"])
    route = gn.last_route()
    torch.cuda.synchronize()
    what = f"{route} {dt.__name__} {shape} bias={bias is not None} beta={beta is not None} off={off}"
    assert_close(to_host(out.output).reshape(-1, hidden), ref[0], f"output ({what})")
    if want["sum"]:
        same = assert_bitwise_nan if non_finite else assert_bitwise
        same(to_host(out.input_skip_bias_sum).reshape(-1, hidden), ref[3], f"S ({what})")
    if want["inv"]:
        assert_close(to_host(out.inv_std_var).reshape(-1), ref[2].reshape(-1), f"inv_std_var ({what})")
    if want["mean"]:
        assert_close(to_host(out.mean).reshape(-1), ref[1].reshape(-1), f"mean ({what})")


@pytest.mark.parametrize("case", range(N_CASES))
def test_gated(case):
    gated(np.random.default_rng(2000 + case), False)


@pytest.mark.parametrize("case", range(N_NON_FINITE))
def test_gated_non_finite(case):
    """As test_gated, with infinities and NaNs planted in X and in the gate."""
    gated(np.random.default_rng(5000 + case), True)


def gated(rng, non_finite):
    dt = F16 if rng.random() < 0.6 else F32
    C = draw_length(rng, [(1, 64, 3), (65, 1024, 4), (1025, 9000, 2), (9001, 40000, 1)])
    rows = int(rng.integers(1, max(2, min(400, MAX_ELEMS // C)) + 1))
    X, G = normal(rng, (rows, C), dt), normal(rng, (rows, C), dt)
    scale = uniform(rng, C, dt)
    if non_finite:
        plant(rng, X, None, dt, int(rng.integers(1, 4)))
        plant(rng, G, None, dt, int(rng.integers(0, 3)))
    off = int(rng.choice([0, 0, 0, 1, 2, 4]))
    ref = oracle.gated_rms_norm(X, scale, G, 1e-5)
    Y = gn.gated_rms_norm(dev(X, off), dev(scale), dev(G, off), 1e-5)
    route = gn.last_route()
    torch.cuda.synchronize()
    assert_close(to_host(Y), ref, f"Y ({route} {dt.__name__} rows={rows} C={C} off={off})")


@pytest.mark.parametrize("case", range(N_CASES))
def test_skip_group_norm(case):
    skip_group_norm(np.random.default_rng(3000 + case), False)


@pytest.mark.parametrize("case", range(N_NON_FINITE))
def test_skip_group_norm_non_finite(case):
    """As test_skip_group_norm, with infinities, NaNs and overflowing sums planted in X (and skip)."""
    skip_group_norm(np.random.default_rng(6000 + case), True)


def skip_group_norm(rng, non_finite):
    T = F16 if rng.random() < 0.6 else F32
    M = F16 if rng.random() < 0.5 else F32
    groups = int(rng.choice([1, 2, 4, 8, 16, 32]))
    cpg = draw_length(rng, [(1, 8, 2), (9, 48, 3)])
    C = groups * cpg
    N = int(rng.integers(1, 4))
    H, W = int(rng.integers(1, 25)), int(rng.integers(1, 25))
    while N * C * H * W > MAX_ELEMS:
        H = max(1, H // 2)
    cl = int(rng.random() < 0.6)
    shape = (N, H, W, C) if cl else (N, C, H, W)
    X = normal(rng, shape, T)
    bcast = bool(rng.random() < 0.3)
    skip = normal(rng, (N, C), T) if bcast else normal(rng, shape, T)
    gamma, beta = uniform(rng, C, M), normal(rng, C, M, 0.1)
    bias = normal(rng, C, T, 0.1) if rng.random() < 0.5 else None
    if non_finite:
        plant(rng, X, None if bcast else skip, T, int(rng.integers(1, 5)))
    act = int(rng.random() < 0.5)
    want_sum = bool(rng.random() < 0.5)
    off = int(rng.choice([0, 0, 0, 1, 4]))
    ref_y, ref_s = oracle.skip_group_norm(X, gamma, beta, skip, bias, groups=groups, activation=act,
                                          epsilon=1e-5, channels_last=cl, want_sum=True)
    out = gn.skip_group_norm(dev(X, off), dev(gamma), dev(beta), dev(skip), dev(bias), groups=groups,
                             activation=act, epsilon=1e-5, channels_last=cl, want_sum=want_sum)
    route = gn.last_route()
    torch.cuda.synchronize()
    what = (f"{route} {T.__name__}/{M.__name__} {'nhwc' if cl else 'nchw'} {shape} g={groups} "
            f"bcast={bcast} bias={bias is not None} act={act} off={off}")
    assert_close(to_host(out.Y), ref_y, f"Y ({what})")
    if want_sum:
        (assert_bitwise_nan if non_finite else assert_bitwise)(to_host(out.S), ref_s, f"S ({what})")


LARGE_SGN_CASES = 48


@pytest.mark.parametrize("case", range(LARGE_SGN_CASES))
def test_skip_group_norm_large(case):
    """Larger images (H, W up to 128, up to 4M elements a tensor), so that
    NHWC and NCHW groups spread over several workgroups (cluster exchanges),
    the split routes and packed runs of pixels whose channels are not a
    whole number of vectors (odd C) are drawn; all tensors 16-byte
    aligned, so the vector and packed routes apply wherever their shapes
    allow."""
    rng = np.random.default_rng(4000 + case)
    T = F16 if rng.random() < 0.6 else F32
    M = F16 if rng.random() < 0.5 else F32
    groups = int(rng.choice([1, 3, 5, 8, 16, 32]))
    cpg = draw_length(rng, [(1, 3, 2), (4, 16, 3), (17, 40, 2)])
    C = groups * cpg
    N = int(rng.integers(1, 5))
    H, W = int(rng.integers(8, 129)), int(rng.integers(8, 129))
    while N * C * H * W > 2 * MAX_ELEMS:
        H = max(1, H // 2)
    cl = int(rng.random() < 0.6)
    shape = (N, H, W, C) if cl else (N, C, H, W)
    X = normal(rng, shape, T)
    bcast = bool(rng.random() < 0.3)
    skip = normal(rng, (N, C), T) if bcast else normal(rng, shape, T)
    gamma, beta = uniform(rng, C, M), normal(rng, C, M, 0.1)
    bias = normal(rng, C, T, 0.1) if rng.random() < 0.5 else None
    act = int(rng.random() < 0.5)
    want_sum = bool(rng.random() < 0.6)
    ref_y, ref_s = oracle.skip_group_norm(X, gamma, beta, skip, bias, groups=groups, activation=act,
                                          epsilon=1e-5, channels_last=cl, want_sum=True)
    out = gn.skip_group_norm(dev(X), dev(gamma), dev(beta), dev(skip), dev(bias), groups=groups,
                             activation=act, epsilon=1e-5, channels_last=cl, want_sum=want_sum)
    route = gn.last_route()
    torch.cuda.synchronize()
    print(f"case {case}: {route}")
    what = (f"{route} {T.__name__}/{M.__name__} {'nhwc' if cl else 'nchw'} {shape} g={groups} "
            f"bcast={bcast} bias={bias is not None} act={act}")
    assert_close(to_host(out.Y), ref_y, f"Y ({what})")
    if want_sum:
        assert_bitwise(to_host(out.S), ref_s, f"S ({what})")


BATCHED_NHWC_CASES = 24


@pytest.mark.parametrize("case", range(BATCHED_NHWC_CASES))
def test_skip_group_norm_batched_nhwc(case):
    """Batches of 6-16 NHWC images whose pixels are not a whole number of
    16-byte vectors (C times the element size not a multiple of 16), widths
    mostly a multiple of 8: grids large enough for the cluster over packed
    runs of pixels, beside element and narrow accesses and the split route
    where the plan sends them."""
    rng = np.random.default_rng(7000 + case)
    T = F16 if rng.random() < 0.6 else F32
    size = np.dtype(T).itemsize
    M = F16 if rng.random() < 0.5 else F32
    groups = int(rng.choice([1, 3, 5, 7, 12, 15]))
    cpg = int(rng.integers(1, 9))
    for _ in range(4):
        if groups * cpg * size % 16:
            break
        cpg += 1
    C = groups * cpg
    N = int(rng.integers(6, 17))
    H = int(rng.integers(24, 97))
    W = 8 * int(rng.integers(3, 13)) if rng.random() < 0.8 else int(rng.integers(24, 97))
    while N * C * H * W > 2 * MAX_ELEMS:
        H = max(1, H // 2)
    shape = (N, H, W, C)
    X = normal(rng, shape, T)
    bcast = bool(rng.random() < 0.3)
    skip = normal(rng, (N, C), T) if bcast else normal(rng, shape, T)
    gamma, beta = uniform(rng, C, M), normal(rng, C, M, 0.1)
    bias = normal(rng, C, T, 0.1) if rng.random() < 0.5 else None
    act = int(rng.random() < 0.5)
    want_sum = bool(rng.random() < 0.6)
    ref_y, ref_s = oracle.skip_group_norm(X, gamma, beta, skip, bias, groups=groups, activation=act,
                                          epsilon=1e-5, channels_last=1, want_sum=True)
    out = gn.skip_group_norm(dev(X), dev(gamma), dev(beta), dev(skip), dev(bias), groups=groups,
                             activation=act, epsilon=1e-5, channels_last=1, want_sum=want_sum)
    route = gn.last_route()
    torch.cuda.synchronize()
    print(f"case {case}: {route}")
    what = (f"{route} {T.__name__}/{M.__name__} nhwc {shape} g={groups} bcast={bcast} "
            f"bias={bias is not None} act={act}")
    assert_close(to_host(out.Y), ref_y, f"Y ({what})")
    if want_sum:
        assert_bitwise(to_host(out.S), ref_s, f"S ({what})")
