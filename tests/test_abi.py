"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects every invalid call during host validation, before any
HIP call.  Pointers here are fake addresses that are never dereferenced: each
call is built to fail validation (or to have zero elements, which launches
nothing).  Skipped when a GPU is visible, so that no bug in validation could
ever launch a kernel on a fake address."""
import ctypes
import os
import re
import subprocess
import threading

import pytest
import torch

from group_normalization_amd import _lib
from group_normalization_amd._lib import SN_BF16, SN_F16, SN_F32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skipnorm.h")

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-pointer validation tests run only without a GPU")

OK, NULL, DTYPE, SHAPE, ATTR, ALIAS, WORKSPACE, HIP = range(8)
A = 0x10000000  # fake, 16-byte aligned, never dereferenced
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert getattr(lib, name) is not None


def test_abi_version(lib):
    assert lib.skipnorm_abi_version() == 2


def err(lib):
    return lib.skipnorm_last_error().decode()


# ------------------------------------------------------------------ SSLN
def ssln(lib, T=SN_F32, rows=4, hidden=8, inp=A, skip=A + MB, gamma=A + 2 * MB, bias=None,
         eps=1e-6, out=A + 3 * MB, mean=None, inv=None, s=None):
    return lib.skip_rms_norm(T, rows, hidden, inp, skip, gamma, bias, eps, out, mean, inv, s, None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(T=SN_BF16), DTYPE, "bfloat16"),
    (dict(T=9), DTYPE, "unknown dtype"),
    (dict(hidden=0), SHAPE, "hidden"),
    (dict(rows=-1), SHAPE, "rows"),
    (dict(hidden=(1 << 30) + 1), SHAPE, "hidden"),
    (dict(eps=-1e-6), ATTR, "epsilon"),
    (dict(eps=float("nan")), ATTR, "epsilon"),
    (dict(eps=float("inf")), ATTR, "epsilon"),
    (dict(gamma=None), NULL, "gamma"),
    (dict(inp=None), NULL, "required"),
    (dict(out=None), NULL, "required"),
    (dict(out=A + 8), ALIAS, "output overlaps input input"),
    (dict(s=A + 3 * MB + 16), ALIAS, "overlaps output"),
    (dict(mean=A + 5 * MB, inv=A + 5 * MB + 4), ALIAS, "mean overlaps output inv_std_var"),
    (dict(bias=A + 3 * MB + 4), ALIAS, "overlaps input bias"),
])
def test_ssln_rejects(lib, kw, status, text):
    assert ssln(lib, **kw) == status
    assert text in err(lib)


def test_ssln_zero_rows_is_a_no_op(lib):
    assert ssln(lib, rows=0, inp=None, skip=None, out=None) == OK
    assert err(lib) == ""
    assert lib.skipnorm_last_route() == b"ssln.empty"


# ------------------------------------------------------------------ SkipLayerNorm
def sln(lib, T=SN_F32, rows=4, hidden=8, inp=A, skip=A + MB, gamma=A + 2 * MB, beta=None, bias=None,
        eps=1e-6, out=A + 3 * MB, mean=None, inv=None, s=None):
    return lib.skip_layer_norm(T, rows, hidden, inp, skip, gamma, beta, bias, eps, out, mean, inv, s,
                               None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(T=SN_BF16), DTYPE, "bfloat16"),
    (dict(hidden=0), SHAPE, "skip_layer_norm: need rows >= 0"),
    (dict(eps=-1e-6), ATTR, "epsilon"),
    (dict(gamma=None), NULL, "skip_layer_norm: gamma"),
    (dict(inp=None), NULL, "required"),
    (dict(beta=A + 3 * MB + 8), ALIAS, "output overlaps input beta"),
    (dict(s=A + 3 * MB + 16), ALIAS, "overlaps output"),
])
def test_sln_rejects(lib, kw, status, text):
    assert sln(lib, **kw) == status
    assert text in err(lib)


def test_sln_zero_rows_is_a_no_op(lib):
    assert sln(lib, rows=0, inp=None, skip=None, out=None) == OK
    assert err(lib) == ""
    assert lib.skipnorm_last_route() == b"ssln.empty"


# ------------------------------------------------------------------ Gated
def gated(lib, T=SN_F16, numel=64, span=16, X=A, scale=A + MB, gate=A + 2 * MB, eps=1e-5,
          Y=A + 3 * MB):
    return lib.gated_rms_norm(T, numel, span, X, scale, gate, eps, Y, None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(T=SN_BF16), DTYPE, "bfloat16"),
    (dict(numel=60, span=16), SHAPE, "not a multiple of the span"),
    (dict(span=0), SHAPE, "span"),
    (dict(numel=-16), SHAPE, "numel"),
    (dict(eps=-1.0), ATTR, "epsilon"),
    (dict(scale=None), NULL, "scale"),
    (dict(gate=None), NULL, "required"),
    (dict(Y=A + 2 * MB + 64), ALIAS, "Y overlaps input gate"),
    (dict(Y=A + MB), ALIAS, "Y overlaps input scale"),
])
def test_gated_rejects(lib, kw, status, text):
    assert gated(lib, **kw) == status
    assert text in err(lib)


def test_gated_zero_rows_is_a_no_op(lib):
    assert gated(lib, numel=0, X=None, gate=None, Y=None) == OK


# ------------------------------------------------------------------ SGN
def ws_size(lib, T=SN_F16, N=2, C=320, H=64, W=64, groups=32, cl=1):
    out = ctypes.c_size_t(0)
    st = lib.skip_group_norm_workspace_size(T, N, C, H, W, groups, cl, ctypes.byref(out))
    return st, out.value


def sgn(lib, T=SN_F16, M=SN_F32, N=2, C=32, H=4, W=4, X=A, gamma=A + MB, beta=A + 2 * MB,
        skip=A + 3 * MB, bcast=0, bias=None, eps=1e-5, groups=8, cl=1, act=0, Y=A + 4 * MB,
        S=None, ws=A + 6 * MB, ws_bytes=1 << 20):
    return lib.skip_group_norm(T, M, N, C, H, W, X, gamma, beta, skip, bcast, bias, eps, groups, cl,
                               act, Y, S, ws, ws_bytes, None)


def test_workspace_size(lib):
    st, n4 = ws_size(lib)
    assert st == OK and n4 > 0
    st, n5 = ws_size(lib, T=SN_F32, N=4, C=1280, H=32, W=32, cl=0)
    assert st == OK and n5 > 0
    assert ws_size(lib, N=0) == (OK, 0)
    assert ws_size(lib, H=0) == (OK, 0)
    assert ws_size(lib, groups=7)[0] == ATTR
    assert ws_size(lib, T=SN_BF16)[0] == DTYPE
    assert lib.skip_group_norm_workspace_size(SN_F16, 1, 8, 1, 1, 2, 1, None) == NULL


@pytest.mark.parametrize("kw,status,text", [
    (dict(T=SN_BF16), DTYPE, "bfloat16"),
    (dict(M=SN_BF16), DTYPE, "gamma/beta"),
    (dict(groups=7), ATTR, "divide C"),
    (dict(groups=0), ATTR, "groups"),
    (dict(act=2), ATTR, "activation"),
    (dict(act=-1), ATTR, "activation"),
    (dict(eps=-1e-5), ATTR, "epsilon"),
    (dict(C=0), SHAPE, "C >= 1"),
    (dict(N=-1), SHAPE, "N, H, W"),
    (dict(C=1 << 12, H=1 << 10, W=1 << 9, groups=1), SHAPE, "2^30"),
    (dict(gamma=None), NULL, "gamma and beta"),
    (dict(skip=None), NULL, "required"),
    (dict(Y=None), NULL, "required"),
    (dict(ws=None), WORKSPACE, "NULL"),
    (dict(ws_bytes=16), WORKSPACE, "required"),
    (dict(ws=A + 6 * MB + 4), WORKSPACE, "aligned"),
    (dict(Y=A + 64), ALIAS, "Y overlaps input X"),
    (dict(S=A + 4 * MB + 2), ALIAS, "Y overlaps output S"),
    (dict(ws=A + 3 * MB), ALIAS, "workspace overlaps input skip"),
    (dict(bias=A + 4 * MB), ALIAS, "Y overlaps input bias"),
])
def test_sgn_rejects(lib, kw, status, text):
    assert sgn(lib, **kw) == status
    assert text in err(lib)


def test_sgn_empty_is_a_no_op(lib):
    assert sgn(lib, N=0, X=None, skip=None, Y=None, ws=None, ws_bytes=0) == OK
    assert sgn(lib, H=0, X=None, skip=None, Y=None, ws=None, ws_bytes=0) == OK


def sgn_noalloc(lib, T=SN_F16, M=SN_F32, N=2, C=32, H=4, W=4, X=A, gamma=A + MB, beta=A + 2 * MB,
                skip=A + 3 * MB, bcast=0, bias=None, eps=1e-5, groups=8, cl=1, act=0, Y=A + 4 * MB,
                S=None):
    return lib.skip_group_norm_noalloc(T, M, N, C, H, W, X, gamma, beta, skip, bcast, bias, eps,
                                       groups, cl, act, Y, S, None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(T=SN_BF16), DTYPE, "bfloat16"),
    (dict(groups=7), ATTR, "divide C"),
    (dict(act=2), ATTR, "activation"),
    (dict(gamma=None), NULL, "gamma and beta"),
    (dict(Y=None), NULL, "required"),
    (dict(Y=A + 64), ALIAS, "Y overlaps input X"),
    # 32 x 1280 x 512 x 512 float32 NCHW needs ~42 MB of partials: more than
    # the static scratch's 8 MiB.
    (dict(T=SN_F32, N=32, C=1280, H=512, W=512, groups=32, cl=0, gamma=A + (1 << 36),
          beta=A + (1 << 36) + MB, skip=A + (1 << 37), bcast=1, Y=A + (1 << 38)),
     WORKSPACE, "static scratch holds 8388608"),
])
def test_sgn_noalloc_rejects(lib, kw, status, text):
    assert sgn_noalloc(lib, **kw) == status
    assert text in err(lib)


def test_sgn_noalloc_empty_is_a_no_op(lib):
    assert sgn_noalloc(lib, N=0, X=None, skip=None, Y=None) == OK
    assert sgn_noalloc(lib, H=0, X=None, skip=None, Y=None) == OK


# ------------------------------------------------------------------ hooks
def test_force_route_round_trip(lib):
    assert lib.skipnorm_force_route(1) == 0
    assert lib.skipnorm_force_route(7) == 1   # unknown: unchanged, reports current
    assert lib.skipnorm_force_route(-1) == 1
    assert lib.skipnorm_force_route(5) == 1   # the flat GatedRMSNorm route
    assert lib.skipnorm_force_route(6) == 5
    assert lib.skipnorm_force_route(0) == 5


def test_last_error_is_per_thread(lib):
    assert ssln(lib, hidden=0) == SHAPE
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
