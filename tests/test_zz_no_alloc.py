"""skip_group_norm_noalloc (the entry point for callers that cannot allocate
device memory) against skip_group_norm with a caller's workspace, called
through the C ABI with raw pointers.

Both entry points run the same kernels with the same arithmetic, so their
outputs must agree bit for bit (stricter than the oracle tolerance); the
oracle is checked as well.  Each test makes consecutive calls into the one
static scratch array, the later ones on smaller inputs, so a call that read
what the previous call left behind would show."""
import ctypes

import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
import workloads
from group_normalization_amd import _lib
from parity import assert_bitwise, assert_close, desc, to_dev, to_host

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 8 << 20
WORKSPACE = 6


def noalloc_call(x, a, want_sum):
    """skip_group_norm_noalloc through ctypes; outputs allocated here, the
    library allocates nothing."""
    X = x["X"]
    Y = torch.empty_like(X)
    S = torch.empty_like(X) if want_sum else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = _lib.lib().skip_group_norm_noalloc(
        desc(X), desc(x["gamma"]), desc(x["beta"]), desc(x["skip"]), desc(x.get("bias")),
        float(a["epsilon"]), int(a["groups"]), 1 if a["channels_last"] else 0, int(a["activation"]),
        desc(Y), desc(S), stream)
    _lib.check(st)
    return Y, S


def workspace_call(x, a, want_sum):
    out = gn.skip_group_norm(x["X"], x["gamma"], x["beta"], x["skip"], x.get("bias"),
                             groups=a["groups"], activation=a["activation"], epsilon=a["epsilon"],
                             channels_last=a["channels_last"], want_sum=want_sum)
    return out.Y, out.S


CASES = [
    # (N, C, H, W, T, M, channels_last, broadcast, bias, groups, activation, want_sum)
    (2, 320, 64, 64, np.float16, np.float32, 1, False, True, 32, 1, True),   # the NHWC workload
    (4, 1280, 32, 32, np.float32, np.float16, 0, True, False, 32, 0, False),  # the NCHW workload
    (2, 640, 16, 16, np.float16, np.float16, 0, False, True, 32, 1, True),
    (1, 320, 8, 8, np.float32, np.float32, 1, True, False, 16, 0, True),
    (1, 64, 7, 9, np.float16, np.float32, 0, False, True, 8, 1, True),        # odd plane: phased
    (2, 15, 16, 16, np.float16, np.float32, 1, False, True, 5, 1, True),     # odd C: element accesses (split: packed runs)
    (1, 15, 512, 512, np.float16, np.float32, 1, False, True, 5, 1, True),   # packed runs, finalize launch
    (8, 15, 64, 128, np.float16, np.float32, 1, False, True, 5, 1, True),    # the cluster over packed runs
]


def inputs(case, seed):
    N, C, H, W, T, M, cl, bc, bias, groups, act, want_sum = case
    w = workloads.sgn("noalloc", N, C, H, W, T, M, channels_last=bool(cl), broadcast_skip=bc,
                      bias=bias, groups=groups, activation=act, epsilon=1e-5)
    host = workloads.generate(w, seed)
    return host, {k: to_dev(v) for k, v in host.items()}, w.attrs, want_sum


def check_pair(case, seed):
    host, dev, a, want_sum = inputs(case, seed)
    y0, s0 = noalloc_call(dev, a, want_sum)
    route = gn.last_route()
    y1, s1 = workspace_call(dev, a, want_sum)
    assert gn.last_route() == route
    assert_bitwise(to_host(y0), to_host(y1), f"Y {case}")
    if want_sum:
        assert_bitwise(to_host(s0), to_host(s1), f"S {case}")
    ry, rs = oracle.skip_group_norm(host["X"], host["gamma"], host["beta"], host["skip"],
                                    host.get("bias"), groups=a["groups"], activation=a["activation"],
                                    epsilon=a["epsilon"], channels_last=a["channels_last"],
                                    want_sum=want_sum)
    assert_close(to_host(y0), ry, f"Y vs oracle {case}")
    if want_sum:
        assert_bitwise(to_host(s0), rs, f"S vs oracle {case}")
    return route


def test_noalloc_two_calls_second_smaller():
    # The NHWC workload, then a much smaller NCHW one into the same scratch.
    r0 = check_pair(CASES[0], seed=0)
    r1 = check_pair(CASES[3], seed=1)
    assert r0.startswith("sgn.cluster.nhwc") and r1.startswith("sgn.")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:4])) + ("nhwc" if c[6] else "nchw"))
def test_noalloc_matches_workspace_entry_point(case):
    check_pair(case, seed=2)
    check_pair(case, seed=3)  # again: the scratch now holds this shape's last call


@pytest.mark.parametrize("route", ["split", "block"])
def test_noalloc_split_routes(route):
    # The three-launch routes keep their partials and (mean, rstd) in the scratch.
    with gn.force_route(route):
        r0 = check_pair(CASES[2], seed=4)
        r1 = check_pair(CASES[4], seed=5)
        r2 = check_pair(CASES[5], seed=6)  # odd C: packed runs with the finalize folded (split)
    assert r0.startswith("sgn.split") and r1.startswith("sgn.split") and r2.startswith("sgn.split")
    if route == "split":
        assert r2 == "sgn.split.nhwc.packed.fold.vec16"


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # NCHW float32 32 x 1280 x 512 x 512 with 32 groups needs ~42 MB of
    # partials; the call is rejected during validation, before anything is
    # enqueued (the small tensors behind the descriptors are never touched).
    xs = (32, 1280, 512, 512)
    need = ctypes.c_size_t()
    _lib.check(_lib.lib().skip_group_norm_workspace_size(_lib.tensor_desc(None, _lib.SN_F32, xs), 32, 0,
                                                         ctypes.byref(need)))
    assert need.value > SCRATCH_BYTES
    x = torch.empty(16, device="cuda")
    y = torch.empty(16, device="cuda")
    big = _lib.tensor_desc(x.data_ptr(), _lib.SN_F32, xs)
    out = _lib.tensor_desc(y.data_ptr(), _lib.SN_F32, xs)
    par = _lib.tensor_desc(x.data_ptr(), _lib.SN_F32, (1280,))
    skp = _lib.tensor_desc(x.data_ptr(), _lib.SN_F32, (32, 1280))
    st = _lib.lib().skip_group_norm_noalloc(big, par, par, skp, None, 1e-5, 32, 0, 0, out, None, None)
    assert st == WORKSPACE
    assert "static scratch" in _lib.lib().skipnorm_last_error().decode()


def test_noalloc_binding_matches():
    # The Python binding of the same entry point, with caller-provided outputs.
    host, dev, a, want_sum = inputs(CASES[0], seed=6)
    Y = torch.empty_like(dev["X"])
    S = torch.empty_like(dev["X"])
    out = gn.skip_group_norm_noalloc(dev["X"], dev["gamma"], dev["beta"], dev["skip"], dev["bias"],
                                     groups=a["groups"], activation=a["activation"], Y=Y, S=S,
                                     epsilon=a["epsilon"], channels_last=a["channels_last"])
    assert out.Y is Y and out.S is S
    y1, s1 = workspace_call(dev, a, True)
    assert_bitwise(to_host(Y), to_host(y1), "Y")
    assert_bitwise(to_host(S), to_host(s1), "S")
