"""The C-ABI library on the CPU: it loads, exports every symbol the headers
declare, and rejects every invalid call during host validation, before any
HIP call: ranks, shapes and element types of every tensor descriptor against
the operator contracts, attributes, pointers, aliasing and workspace sizes.
Pointers here are fake addresses that are never dereferenced: each call is
built to fail validation (or to have zero elements, which launches nothing).
Skipped when a GPU is visible, so that no bug in validation could ever launch
a kernel on a fake address.

Validation accepts tensors at any element-aligned address, and some routes
then read past a tensor's ends.  For rows, NCHW groups or flat row streams
off the 16-byte grid, the phased and flat routes read whole aligned 16-byte
vectors. Those reads can touch up to 15 bytes beside a tensor's first and
last element, inside the same aligned block. A bounds-checked CPU emulation
of those kernels would flag the reads. On the GPU they cannot fault,
because device memory is mapped in pages. The read bytes only ever fill
lanes that are masked out. That nothing outside the outputs is written is
checked on the GPU with guard elements around every output (test_phased_rows
and test_flat_rows_off_the_grid in test_gpu_ssln.py, test_nchw_phased_groups
in test_gpu_sgn.py, test_flat_route in test_gpu_gated.py)."""
import ctypes
import os
import re
import subprocess
import threading

import pytest
import torch

from group_normalization_amd import _lib
from group_normalization_amd._lib import SN_BF16, SN_F16, SN_F32, tensor_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("skipnorm.h", "skipnorm_testing.h")]

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-pointer validation tests run only without a GPU")

OK, NULL, DTYPE, SHAPE, ATTR, ALIAS, WORKSPACE, HIP = range(8)
A = 0x10000000  # fake, 16-byte aligned, never dereferenced
MB = 1 << 20
GB = 1 << 30
ABSENT = object()


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text))
    return sorted(names)


def test_headers_declare_the_abi():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert getattr(lib, name) is not None


def test_abi_version(lib):
    assert lib.skipnorm_abi_version() == 3


def test_descriptor_layout_matches_the_header():
    # sn_tensor_in / sn_tensor_out: pointer, enum, int32 rank, int64 shape[8].
    assert ctypes.sizeof(_lib.TensorDesc) == 8 + 4 + 4 + 8 * 8
    assert _lib.TensorDesc.shape.offset == 16


def err(lib):
    return lib.skipnorm_last_error().decode()


def T(ptr, dtype, shape):
    return tensor_desc(ptr, dtype, shape)


def pick(value, default):
    """A keyword's value: ABSENT -> None (no descriptor), None -> default."""
    if value is ABSENT:
        return None
    return default if value is None else value


# ------------------------------------------------------------------ SSLN
def ssln(lib, dt=SN_F32, shape=(4, 8), inp=None, skip=None, gamma=None, bias=ABSENT, eps=1e-6,
         out=None, mean=ABSENT, inv=ABSENT, s=ABSENT, layer=False, beta=ABSENT):
    hidden = shape[-1]
    stat = tuple(shape[:-1]) + (1,)
    args = [pick(inp, T(A, dt, shape)), pick(skip, T(A + GB, dt, shape)),
            pick(gamma, T(A + 2 * GB, dt, (hidden,)))]
    if layer:
        args.append(pick(beta, T(A + 2 * GB + MB, dt, (hidden,))) if beta is not ABSENT else None)
    args += [pick(bias, T(A + 2 * GB + 2 * MB, dt, (hidden,))) if bias is not ABSENT else None, eps,
             pick(out, T(A + 3 * GB, dt, shape)),
             pick(mean, T(A + 4 * GB, SN_F32, stat)) if mean is not ABSENT else None,
             pick(inv, T(A + 4 * GB + MB, SN_F32, stat)) if inv is not ABSENT else None,
             pick(s, T(A + 5 * GB, dt, shape)) if s is not ABSENT else None, None]
    return (lib.skip_layer_norm if layer else lib.skip_rms_norm)(*args)


@pytest.mark.parametrize("kw,status,text", [
    # element types
    (dict(dt=SN_BF16), DTYPE, "input: bfloat16"),
    (dict(dt=9), DTYPE, "unknown dtype"),
    (dict(skip=T(A + GB, SN_F16, (4, 8))), DTYPE, "skip must be float32"),
    (dict(gamma=T(A + 2 * GB, SN_F16, (8,))), DTYPE, "gamma must be float32"),
    (dict(bias=T(A + 2 * GB, SN_BF16, (8,))), DTYPE, "bias: bfloat16"),
    (dict(out=T(A + 3 * GB, SN_F16, (4, 8))), DTYPE, "output must be float32"),
    (dict(dt=SN_F16, inv=T(A + 4 * GB, SN_F16, (4, 1))), DTYPE, "inv_std_var must be float32"),
    (dict(s=T(A + 5 * GB, SN_F16, (4, 8))), DTYPE, "input_skip_bias_sum must be float32"),
    # ranks and shapes
    (dict(shape=(32,)), SHAPE, "input must have rank 2"),
    (dict(shape=(2, 2, 2, 8)), SHAPE, "input must have rank 2"),
    (dict(shape=(4, 0)), SHAPE, "hidden"),
    (dict(shape=(4, (1 << 30) + 1)), SHAPE, "hidden"),
    (dict(inp=T(A, SN_F32, (4, -8))), SHAPE, "negative extent"),
    (dict(inp=T(A, SN_F32, (1 << 24, 1 << 24))), SHAPE, "2^46"),
    (dict(skip=T(A + GB, SN_F32, (4, 9))), SHAPE, "skip must have shape (4, 8)"),
    (dict(skip=T(A + GB, SN_F32, (32,))), SHAPE, "skip must have shape (4, 8)"),
    (dict(gamma=T(A + 2 * GB, SN_F32, (9,))), SHAPE, "gamma must have shape (8,)"),
    (dict(gamma=T(A + 2 * GB, SN_F32, (1, 8))), SHAPE, "gamma must have shape (8,)"),
    (dict(bias=T(A + 2 * GB, SN_F32, (4,))), SHAPE, "bias must have shape (8,)"),
    (dict(out=T(A + 3 * GB, SN_F32, (8, 4))), SHAPE, "output must have shape (4, 8)"),
    (dict(s=T(A + 5 * GB, SN_F32, (4, 8, 1))), SHAPE, "input_skip_bias_sum must have shape"),
    (dict(mean=T(A + 4 * GB, SN_F32, (4,))), SHAPE, "mean must have shape (4, 1)"),
    (dict(shape=(2, 3, 8), inv=T(A + 4 * GB, SN_F32, (6, 1))), SHAPE, "inv_std_var must have shape (2, 3, 1)"),
    # attributes
    (dict(eps=-1e-6), ATTR, "epsilon"),
    (dict(eps=float("nan")), ATTR, "epsilon"),
    (dict(eps=float("inf")), ATTR, "epsilon"),
    # required tensors and pointers
    (dict(gamma=ABSENT), NULL, "gamma is required"),
    (dict(inp=ABSENT), NULL, "input is required"),
    (dict(out=ABSENT), NULL, "output is required"),
    (dict(inp=T(None, SN_F32, (4, 8))), NULL, "input has 32 elements and a NULL data pointer"),
    (dict(gamma=T(None, SN_F32, (8,))), NULL, "gamma has 8 elements"),
    # aliasing
    (dict(out=T(A + 8, SN_F32, (4, 8))), ALIAS, "output output overlaps input input"),
    (dict(s=T(A + 3 * GB + 16, SN_F32, (4, 8))), ALIAS, "overlaps output"),
    (dict(mean=T(A + 8, SN_F32, (4, 1))), ALIAS, "output mean overlaps input input"),
    (dict(mean=T(A + 6 * GB, SN_F32, (4, 1)), inv=T(A + 6 * GB + 4, SN_F32, (4, 1))), ALIAS,
     "mean overlaps output inv_std_var"),
    (dict(bias=T(A + 3 * GB + 4, SN_F32, (8,))), ALIAS, "overlaps input bias"),
])
def test_ssln_rejects(lib, kw, status, text):
    assert ssln(lib, **kw) == status
    assert text in err(lib)


def test_ssln_zero_rows_is_a_no_op(lib):
    for shape in ((0, 8), (0, 5, 8), (3, 0, 8)):
        assert ssln(lib, shape=shape, inp=T(None, SN_F32, shape), skip=T(None, SN_F32, shape),
                    out=T(None, SN_F32, shape)) == OK
        assert err(lib) == ""
        assert lib.skipnorm_last_route() == b"ssln.empty"


# ------------------------------------------------------------------ SkipLayerNorm
@pytest.mark.parametrize("kw,status,text", [
    (dict(dt=SN_BF16), DTYPE, "bfloat16"),
    (dict(shape=(4, 0)), SHAPE, "skip_layer_norm: hidden"),
    (dict(beta=T(A + 2 * GB + MB, SN_F32, (7,))), SHAPE, "beta must have shape (8,)"),
    (dict(beta=T(A + 2 * GB + MB, SN_F16, (8,))), DTYPE, "beta must be float32"),
    (dict(eps=-1e-6), ATTR, "epsilon"),
    (dict(gamma=ABSENT), NULL, "skip_layer_norm: gamma is required"),
    (dict(inp=ABSENT), NULL, "required"),
    (dict(beta=T(A + 3 * GB + 8, SN_F32, (8,))), ALIAS, "output output overlaps input beta"),
    (dict(s=T(A + 3 * GB + 16, SN_F32, (4, 8))), ALIAS, "overlaps output"),
])
def test_sln_rejects(lib, kw, status, text):
    assert ssln(lib, layer=True, **kw) == status
    assert text in err(lib)


def test_sln_zero_rows_is_a_no_op(lib):
    assert ssln(lib, layer=True, shape=(0, 8), inp=T(None, SN_F32, (0, 8)), skip=T(None, SN_F32, (0, 8)),
                out=T(None, SN_F32, (0, 8))) == OK
    assert err(lib) == ""
    assert lib.skipnorm_last_route() == b"ssln.empty"


# ------------------------------------------------------------------ Gated
def gated(lib, dt=SN_F16, shape=(4, 16), C=16, X=None, scale=None, gate=None, eps=1e-5, Y=None):
    return lib.gated_rms_norm(pick(X, T(A, dt, shape)), pick(scale, T(A + GB, dt, (C,))),
                              pick(gate, T(A + 2 * GB, dt, shape)), eps,
                              pick(Y, T(A + 3 * GB, dt, shape)), None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(dt=SN_BF16), DTYPE, "bfloat16"),
    (dict(gate=T(A + 2 * GB, SN_F32, (4, 16))), DTYPE, "gate must be float16"),
    (dict(scale=T(A + GB, SN_F32, (16,))), DTYPE, "scale must be float16"),
    (dict(Y=T(A + 3 * GB, SN_F32, (4, 16))), DTYPE, "Y must be float16"),
    (dict(shape=(60,), C=16), SHAPE, "not a multiple of the span"),
    (dict(shape=()), SHAPE, "X must have rank >= 1"),
    (dict(C=0), SHAPE, "span"),
    (dict(scale=T(A + GB, SN_F16, (2, 8))), SHAPE, "scale must be a vector"),
    (dict(scale=T(A + GB, SN_F16, ())), SHAPE, "scale must be a vector"),
    (dict(X=T(A, SN_F16, (4, -16))), SHAPE, "negative extent"),
    (dict(gate=T(A + 2 * GB, SN_F16, (64,))), SHAPE, "gate must have shape (4, 16)"),
    (dict(Y=T(A + 3 * GB, SN_F16, (16, 4))), SHAPE, "Y must have shape (4, 16)"),
    (dict(eps=-1.0), ATTR, "epsilon"),
    (dict(scale=ABSENT), NULL, "scale is required"),
    (dict(gate=ABSENT), NULL, "gate is required"),
    (dict(X=T(None, SN_F16, (4, 16))), NULL, "NULL data pointer"),
    (dict(Y=T(A + 2 * GB + 64, SN_F16, (4, 16))), ALIAS, "Y overlaps input gate"),
    (dict(Y=T(A + GB, SN_F16, (4, 16))), ALIAS, "Y overlaps input scale"),
])
def test_gated_rejects(lib, kw, status, text):
    assert gated(lib, **kw) == status
    assert text in err(lib)


def test_gated_zero_rows_is_a_no_op(lib):
    # Every spelling of a vector scale is accepted.
    for sshape in ((16,), (1, 16), (16, 1), (1, 16, 1)):
        e = T(None, SN_F16, (0, 16))
        assert gated(lib, X=e, gate=e, Y=e, scale=T(A + GB, SN_F16, sshape)) == OK, err(lib)


# ------------------------------------------------------------------ SGN
def x_desc(dt=SN_F16, N=2, C=32, H=4, W=4, cl=1, ptr=A):
    return T(ptr, dt, (N, H, W, C) if cl else (N, C, H, W))


def ws_size(lib, dt=SN_F16, N=2, C=320, H=64, W=64, groups=32, cl=1):
    out = ctypes.c_size_t(0)
    st = lib.skip_group_norm_workspace_size(x_desc(dt, N, C, H, W, cl, ptr=None), groups, cl,
                                            ctypes.byref(out))
    return st, out.value


def sgn_args(dt=SN_F16, M=SN_F32, N=2, C=32, H=4, W=4, cl=1, X=None, gamma=None, beta=None,
             skip=None, bias=ABSENT, eps=1e-5, groups=8, act=0, Y=None, S=ABSENT):
    xs = (N, H, W, C) if cl else (N, C, H, W)
    return [pick(X, T(A, dt, xs)), pick(gamma, T(A + GB, M, (C,))), pick(beta, T(A + GB + MB, M, (C,))),
            pick(skip, T(A + 2 * GB, dt, xs)),
            pick(bias, T(A + GB + 2 * MB, dt, (C,))) if bias is not ABSENT else None, eps, groups, cl,
            act, pick(Y, T(A + 3 * GB, dt, xs)), pick(S, T(A + 4 * GB, dt, xs)) if S is not ABSENT else None]


def sgn(lib, ws=A + 6 * GB, ws_bytes=1 << 20, **kw):
    return lib.skip_group_norm(*sgn_args(**kw), ws, ws_bytes, None)


def sgn_noalloc(lib, **kw):
    return lib.skip_group_norm_noalloc(*sgn_args(**kw), None)


def test_workspace_size(lib):
    st, n4 = ws_size(lib)
    assert st == OK and n4 > 0
    st, n5 = ws_size(lib, dt=SN_F32, N=4, C=1280, H=32, W=32, cl=0)
    assert st == OK and n5 > 0
    assert ws_size(lib, N=0) == (OK, 0)
    assert ws_size(lib, H=0) == (OK, 0)
    assert ws_size(lib, groups=7)[0] == ATTR
    assert ws_size(lib, dt=SN_BF16)[0] == DTYPE
    out = ctypes.c_size_t(0)
    assert lib.skip_group_norm_workspace_size(T(None, SN_F16, (1, 8, 8)), 2, 1, ctypes.byref(out)) == SHAPE
    assert "X must have rank 4" in err(lib)
    assert lib.skip_group_norm_workspace_size(None, 2, 1, ctypes.byref(out)) == NULL
    assert lib.skip_group_norm_workspace_size(x_desc(), 2, 1, None) == NULL


@pytest.mark.parametrize("dt,size,N,C,H,W,groups", [
    (SN_F16, 2, 8, 15, 128, 128, 5), (SN_F16, 2, 1, 15, 512, 512, 5), (SN_F16, 2, 16, 3, 256, 256, 1),
    (SN_F32, 4, 2, 5, 40, 40, 5), (SN_F16, 2, 4, 75, 1024, 1024, 25)])
def test_workspace_size_packed_runs(lib, dt, size, N, C, H, W, groups):
    """NHWC pixels that are not a whole number of 16-byte vectors: the
    workspace holds the packed-run tiling's partials (at least 64 per
    (n, group)) of 16 bytes and one (mean, rstd) pair of 8 bytes per
    (n, group)."""
    from plans import packed_applies, packed_blocks
    assert packed_applies(C, H * W, size)
    B = min(max(packed_blocks(N, C, H * W, size), 64), 16384)
    st, n = ws_size(lib, dt=dt, N=N, C=C, H=H, W=W, groups=groups, cl=1)
    assert st == OK and n == N * groups * B * 16 + N * groups * 8


SGN_REJECTS = [
    # element types
    (dict(dt=SN_BF16), DTYPE, "X: bfloat16"),
    (dict(M=SN_BF16), DTYPE, "gamma: bfloat16"),
    (dict(beta=T(A + GB + MB, SN_F16, (32,))), DTYPE, "beta must be float32 (gamma's type)"),
    (dict(skip=T(A + 2 * GB, SN_F32, (2, 4, 4, 32))), DTYPE, "skip must be float16"),
    (dict(bias=T(A + GB + 2 * MB, SN_F32, (32,))), DTYPE, "bias must be float16"),
    (dict(S=T(A + 4 * GB, SN_F32, (2, 4, 4, 32))), DTYPE, "S must be float16"),
    # ranks and shapes
    (dict(X=T(A, SN_F16, (2, 16, 32))), SHAPE, "X must have rank 4"),
    (dict(C=0, groups=1), SHAPE, "C >= 1"),
    (dict(X=T(A, SN_F16, (-2, 4, 4, 32))), SHAPE, "negative extent"),
    (dict(C=1 << 12, H=1 << 10, W=1 << 9, groups=1), SHAPE, "2^30"),
    (dict(gamma=T(A + GB, SN_F32, (16,))), SHAPE, "gamma must have shape (32,)"),
    (dict(beta=T(A + GB + MB, SN_F32, (1, 32))), SHAPE, "beta must have shape (32,)"),
    (dict(bias=T(A + GB + 2 * MB, SN_F16, (31,))), SHAPE, "bias must have shape (32,)"),
    (dict(Y=T(A + 3 * GB, SN_F16, (2, 32, 4, 4))), SHAPE, "Y must have shape (2, 4, 4, 32)"),
    (dict(skip=T(A + 2 * GB, SN_F16, (2, 33))), SHAPE, "skip must have X's shape"),
    (dict(skip=T(A + 2 * GB, SN_F16, (2, 32, 1, 1))), SHAPE, "skip must have X's shape"),
    (dict(skip=T(A + 2 * GB, SN_F16, (1, 32))), SHAPE, "skip must have X's shape"),
    (dict(skip=T(A + 2 * GB, SN_F16, (64,))), SHAPE, "skip must have X's shape"),
    # attributes
    (dict(groups=7), ATTR, "divide C"),
    (dict(groups=0), ATTR, "groups"),
    (dict(act=2), ATTR, "activation"),
    (dict(act=-1), ATTR, "activation"),
    (dict(eps=-1e-5), ATTR, "epsilon"),
    # required tensors and pointers
    (dict(gamma=ABSENT), NULL, "gamma is required"),
    (dict(beta=ABSENT), NULL, "beta is required"),
    (dict(skip=ABSENT), NULL, "skip is required"),
    (dict(Y=ABSENT), NULL, "Y is required"),
    (dict(X=T(None, SN_F16, (2, 4, 4, 32))), NULL, "X has 1024 elements and a NULL data pointer"),
    # aliasing
    (dict(Y=T(A + 64, SN_F16, (2, 4, 4, 32))), ALIAS, "Y overlaps input X"),
    (dict(S=T(A + 3 * GB + 2, SN_F16, (2, 4, 4, 32))), ALIAS, "Y overlaps output S"),
    (dict(bias=T(A + 3 * GB, SN_F16, (32,))), ALIAS, "Y overlaps input bias"),
]


@pytest.mark.parametrize("kw,status,text", SGN_REJECTS + [
    (dict(ws=None), WORKSPACE, "NULL"),
    (dict(ws_bytes=16), WORKSPACE, "required"),
    (dict(ws=A + 6 * GB + 4), WORKSPACE, "aligned"),
    (dict(ws=A + 2 * GB), ALIAS, "workspace overlaps input skip"),
])
def test_sgn_rejects(lib, kw, status, text):
    assert sgn(lib, **kw) == status
    assert text in err(lib)


@pytest.mark.parametrize("skip_shape", [(2, 32), (2, 1, 1, 32)])
@pytest.mark.parametrize("cl", [0, 1])
def test_sgn_accepts_broadcast_skip_spellings(lib, skip_shape, cl):
    # Both broadcast spellings pass shape validation in both layouts: the
    # call gets as far as the (deliberately missing) workspace.
    assert sgn(lib, cl=cl, skip=T(A + 2 * GB, SN_F16, skip_shape), ws=None) == WORKSPACE
    assert "workspace of" in err(lib)


def test_sgn_empty_is_a_no_op(lib):
    for dims in (dict(N=0), dict(H=0)):
        xs = x_desc(ptr=None, **dims)
        assert sgn(lib, X=xs, skip=xs, Y=xs, ws=None, ws_bytes=0, **dims) == OK, err(lib)


@pytest.mark.parametrize("kw,status,text", SGN_REJECTS[:10] + [
    # 32 x 1280 x 512 x 512 float32 NCHW needs ~42 MB of partials: more than
    # the static scratch's 8 MiB.
    (dict(dt=SN_F32, N=32, C=1280, H=512, W=512, groups=32, cl=0,
          skip=T(A + 2 * GB, SN_F32, (32, 1280))), WORKSPACE, "static scratch holds 8388608"),
])
def test_sgn_noalloc_rejects(lib, kw, status, text):
    assert sgn_noalloc(lib, **kw) == status
    assert text in err(lib)


def test_sgn_noalloc_empty_is_a_no_op(lib):
    for dims in (dict(N=0), dict(H=0)):
        xs = x_desc(ptr=None, **dims)
        assert sgn_noalloc(lib, X=xs, skip=xs, Y=xs, **dims) == OK, err(lib)


# ------------------------------------------------------------------ hooks
def test_force_route_round_trip(lib):
    assert lib.skipnorm_force_route(1) == 0
    assert lib.skipnorm_force_route(7) == 1   # unknown: unchanged, reports current
    assert lib.skipnorm_force_route(-1) == 1
    assert lib.skipnorm_force_route(5) == 1   # the flat GatedRMSNorm route
    assert lib.skipnorm_force_route(6) == 5
    assert lib.skipnorm_force_route(0) == 5


def test_last_error_is_per_thread(lib):
    assert ssln(lib, shape=(4, 0)) == SHAPE
    seen = {}

    def other():
        seen["err"] = err(lib)

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["err"] == ""
    assert "hidden" in err(lib)


def test_copy_rejects(lib):
    assert lib.skipnorm_copy(A, A + MB, 0, None) == OK
    assert lib.skipnorm_copy(A, A + MB, 24, None) == SHAPE
    assert lib.skipnorm_copy(A + 4, A + MB, 32, None) == SHAPE
    assert lib.skipnorm_copy(None, A + MB, 32, None) == NULL
    assert lib.skipnorm_copy(A, A + 16, 64, None) == ALIAS
