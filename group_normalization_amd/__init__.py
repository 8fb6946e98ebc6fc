"""Fused skip-add + normalize operators on AMD Instinct MI355X (gfx950).

Python binding of libskipnorm (C ABI in ``include/skipnorm.h``): argument
marshalling only.  Tensors are torch tensors on a ROCm device; torch provides
device memory and the current stream, and every step of the computation runs
in the library's HIP kernels.  Outputs are allocated here with the shapes
and dtypes the operator contracts define.

Operators (names and defaults follow the ONNX Runtime contrib-op pages):

- ``skip_rms_norm`` -- "com.microsoft.SkipSimplifiedLayerNormalization"
- ``gated_rms_norm`` -- "com.microsoft.GatedRMSNorm"
- ``skip_group_norm`` -- "com.microsoft.SkipGroupNorm"
"""
from __future__ import annotations

import contextlib
import ctypes
from typing import NamedTuple, Optional

import torch

from ._lib import SN_BF16, SN_F16, SN_F32, SkipNormError, check, lib

__all__ = ["skip_layer_norm", "skip_rms_norm", "gated_rms_norm", "skip_group_norm", "skip_group_norm_workspace_size",
           "skip_group_norm_noalloc",
           "SkipRmsNormOutputs", "SkipGroupNormOutputs", "SkipNormError", "force_route",
           "last_route", "exchange_timeout_us", "abi_version", "copy_"]

#: Attribute defaults from the pages' Attributes tables.
SSLN_EPSILON = 9.999999960041972e-13
GATED_EPSILON = 1e-5
SGN_EPSILON = 1e-5

_DTYPES = {torch.float32: SN_F32, torch.float16: SN_F16, torch.bfloat16: SN_BF16}


class SkipRmsNormOutputs(NamedTuple):
    output: torch.Tensor
    mean: Optional[torch.Tensor]
    inv_std_var: Optional[torch.Tensor]
    input_skip_bias_sum: Optional[torch.Tensor]


class SkipGroupNormOutputs(NamedTuple):
    Y: torch.Tensor
    S: Optional[torch.Tensor]


def _code(t: torch.Tensor, what: str) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"{what}: dtype {t.dtype} is not float32/float16") from None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _device_of(*tensors: Optional[torch.Tensor]) -> torch.device:
    present = [t for t in tensors if t is not None]
    dev = present[0].device
    for t in present:
        if t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")
        if not t.is_contiguous():
            raise ValueError("every tensor must be contiguous")
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a ROCm GPU device, not {dev}")
    return dev


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _same_dtype(ref: torch.Tensor, what: str, *tensors: Optional[torch.Tensor]) -> None:
    for t in tensors:
        if t is not None and t.dtype != ref.dtype:
            raise TypeError(f"{what}: all tensors of type T must share {ref.dtype}, got {t.dtype}")


def skip_rms_norm(input: torch.Tensor, skip: torch.Tensor, gamma: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, epsilon: float = SSLN_EPSILON, *,
                  want_mean: bool = False, want_inv_std_var: bool = False,
                  want_sum: bool = False) -> SkipRmsNormOutputs:
    """SkipSimplifiedLayerNormalization over the last axis.

    input/skip: (token_count, hidden) or (batch, sequence, hidden), type T;
    gamma, bias: (hidden,).  Returns (output, mean, inv_std_var,
    input_skip_bias_sum); optional entries are None unless requested.
    """
    if input.dim() not in (2, 3):
        raise ValueError(f"input must have rank 2 or 3, got shape {tuple(input.shape)}")
    if skip.shape != input.shape:
        raise ValueError(f"skip shape {tuple(skip.shape)} != input shape {tuple(input.shape)}")
    hidden = input.shape[-1]
    for name, t in (("gamma", gamma), ("bias", bias)):
        if t is not None and tuple(t.shape) != (hidden,):
            raise ValueError(f"{name} must have shape ({hidden},), got {tuple(t.shape)}")
    _same_dtype(input, "skip_rms_norm", skip, gamma, bias)
    dev = _device_of(input, skip, gamma, bias)
    T = _code(input, "skip_rms_norm")
    rows = input.numel() // hidden if hidden else 0
    output = torch.empty_like(input)
    stat_shape = tuple(input.shape[:-1]) + (1,)
    mean = torch.empty(stat_shape, dtype=torch.float32, device=dev) if want_mean else None
    inv = torch.empty(stat_shape, dtype=torch.float32, device=dev) if want_inv_std_var else None
    s = torch.empty_like(input) if want_sum else None
    with torch.cuda.device(dev):
        check(lib().skip_rms_norm(T, rows, hidden, _ptr(input), _ptr(skip), _ptr(gamma),
                                  _ptr(bias), float(epsilon), _ptr(output), _ptr(mean),
                                  _ptr(inv), _ptr(s), _stream(dev)))
    return SkipRmsNormOutputs(output, mean, inv, s)


def skip_layer_norm(input: torch.Tensor, skip: torch.Tensor, gamma: torch.Tensor,
                    beta: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                    epsilon: float = SSLN_EPSILON, *, want_mean: bool = False,
                    want_inv_std_var: bool = False, want_sum: bool = False) -> SkipRmsNormOutputs:
    """Skip layer normalization with the row mean removed (the non-simplified
    form of SkipSimplifiedLayerNormalization): output = (S - mean) *
    inv_std_var * gamma (+ beta).  Arguments and outputs as skip_rms_norm,
    plus beta (hidden,); mean and inv_std_var are the row mean and inverse
    standard deviation."""
    if input.dim() not in (2, 3):
        raise ValueError(f"input must have rank 2 or 3, got shape {tuple(input.shape)}")
    if skip.shape != input.shape:
        raise ValueError(f"skip shape {tuple(skip.shape)} != input shape {tuple(input.shape)}")
    hidden = input.shape[-1]
    for name, t in (("gamma", gamma), ("beta", beta), ("bias", bias)):
        if t is not None and tuple(t.shape) != (hidden,):
            raise ValueError(f"{name} must have shape ({hidden},), got {tuple(t.shape)}")
    _same_dtype(input, "skip_layer_norm", skip, gamma, beta, bias)
    dev = _device_of(input, skip, gamma, beta, bias)
    T = _code(input, "skip_layer_norm")
    rows = input.numel() // hidden if hidden else 0
    output = torch.empty_like(input)
    stat_shape = tuple(input.shape[:-1]) + (1,)
    mean = torch.empty(stat_shape, dtype=torch.float32, device=dev) if want_mean else None
    inv = torch.empty(stat_shape, dtype=torch.float32, device=dev) if want_inv_std_var else None
    s = torch.empty_like(input) if want_sum else None
    with torch.cuda.device(dev):
        check(lib().skip_layer_norm(T, rows, hidden, _ptr(input), _ptr(skip), _ptr(gamma),
                                    _ptr(beta), _ptr(bias), float(epsilon), _ptr(output),
                                    _ptr(mean), _ptr(inv), _ptr(s), _stream(dev)))
    return SkipRmsNormOutputs(output, mean, inv, s)


def gated_rms_norm(X: torch.Tensor, scale: torch.Tensor, gate: torch.Tensor,
                   epsilon: float = GATED_EPSILON) -> torch.Tensor:
    """GatedRMSNorm: RMS over each contiguous run of C = scale.numel()
    elements of X (rows counted flat), times scale and SiLU(gate)."""
    if X.dim() < 1:
        raise ValueError("X must have rank >= 1")
    if gate.shape != X.shape:
        raise ValueError(f"gate shape {tuple(gate.shape)} != X shape {tuple(X.shape)}")
    if scale.dim() > 1 and max(scale.shape) != scale.numel():
        raise ValueError(f"scale must be a vector ((C), (1, C) or (C, 1)), got {tuple(scale.shape)}")
    _same_dtype(X, "gated_rms_norm", scale, gate)
    dev = _device_of(X, scale, gate)
    Y = torch.empty_like(X)
    with torch.cuda.device(dev):
        check(lib().gated_rms_norm(_code(X, "gated_rms_norm"), X.numel(), scale.numel(), _ptr(X),
                                   _ptr(scale), _ptr(gate), float(epsilon), _ptr(Y), _stream(dev)))
    return Y


def _sgn_dims(X: torch.Tensor, channels_last: int):
    if X.dim() != 4:
        raise ValueError(f"X must have rank 4, got shape {tuple(X.shape)}")
    if channels_last:
        N, H, W, C = X.shape
    else:
        N, C, H, W = X.shape
    return N, C, H, W


def skip_group_norm_workspace_size(X: torch.Tensor, groups: int, channels_last: int = 1) -> int:
    N, C, H, W = _sgn_dims(X, channels_last)
    out = ctypes.c_size_t(0)
    check(lib().skip_group_norm_workspace_size(_code(X, "skip_group_norm"), N, C, H, W, int(groups),
                                               1 if channels_last else 0, ctypes.byref(out)))
    return out.value


def skip_group_norm(X: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, skip: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, *, groups: int, activation: int,
                    epsilon: float = SGN_EPSILON, channels_last: int = 1, want_sum: bool = False,
                    workspace: Optional[torch.Tensor] = None) -> SkipGroupNormOutputs:
    """SkipGroupNorm.  X is (N, H, W, C) when channels_last else (N, C, H, W);
    skip is X's shape or (N, C) / (N, 1, 1, C); gamma/beta (C,) of their own
    type; bias (C,).  ``groups`` and ``activation`` have no default.
    ``workspace`` (uint8, at least skip_group_norm_workspace_size bytes) is
    allocated per call when not given."""
    N, C, H, W = _sgn_dims(X, channels_last)
    if tuple(skip.shape) == tuple(X.shape):
        bcast = 0
    elif tuple(skip.shape) in ((N, C), (N, 1, 1, C)):
        bcast = 1
    else:
        raise ValueError(f"skip shape {tuple(skip.shape)} is neither X's shape {tuple(X.shape)} "
                         f"nor ({N}, {C}) / ({N}, 1, 1, {C})")
    for name, t in (("gamma", gamma), ("beta", beta), ("bias", bias)):
        if t is not None and tuple(t.shape) != (C,):
            raise ValueError(f"{name} must have shape ({C},), got {tuple(t.shape)}")
    _same_dtype(X, "skip_group_norm", skip, bias)
    if beta.dtype != gamma.dtype:
        raise TypeError("gamma and beta must share one dtype (M)")
    dev = _device_of(X, gamma, beta, skip, bias)
    T, M = _code(X, "skip_group_norm"), _code(gamma, "skip_group_norm gamma")
    Y = torch.empty_like(X)
    S = torch.empty_like(X) if want_sum else None
    need = skip_group_norm_workspace_size(X, groups, channels_last)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev:
        raise ValueError("workspace must be on the tensors' device")
    with torch.cuda.device(dev):
        check(lib().skip_group_norm(T, M, N, C, H, W, _ptr(X), _ptr(gamma), _ptr(beta), _ptr(skip),
                                    bcast, _ptr(bias), float(epsilon), int(groups),
                                    1 if channels_last else 0, int(activation), _ptr(Y), _ptr(S),
                                    _ptr(workspace), workspace.numel(), _stream(dev)))
    return SkipGroupNormOutputs(Y, S)


def skip_group_norm_noalloc(X: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
                            skip: torch.Tensor, bias: Optional[torch.Tensor] = None, *, groups: int,
                            activation: int, Y: torch.Tensor, S: Optional[torch.Tensor] = None,
                            epsilon: float = SGN_EPSILON, channels_last: int = 1) -> SkipGroupNormOutputs:
    """skip_group_norm for callers that cannot allocate device memory: the
    caller passes the outputs Y (and S, if wanted), and the library keeps its
    partial moments in its own static scratch (shapes needing more than
    SKIPNORM_NOALLOC_SCRATCH_BYTES are rejected).  Calls that overlap in
    time on one device race on that scratch."""
    N, C, H, W = _sgn_dims(X, channels_last)
    if tuple(skip.shape) == tuple(X.shape):
        bcast = 0
    elif tuple(skip.shape) in ((N, C), (N, 1, 1, C)):
        bcast = 1
    else:
        raise ValueError(f"skip shape {tuple(skip.shape)} is neither X's shape {tuple(X.shape)} "
                         f"nor ({N}, {C}) / ({N}, 1, 1, {C})")
    for name, t in (("gamma", gamma), ("beta", beta), ("bias", bias)):
        if t is not None and tuple(t.shape) != (C,):
            raise ValueError(f"{name} must have shape ({C},), got {tuple(t.shape)}")
    for name, t in (("Y", Y), ("S", S)):
        if t is not None and (tuple(t.shape) != tuple(X.shape) or t.dtype != X.dtype):
            raise ValueError(f"{name} must match X's shape and dtype")
    _same_dtype(X, "skip_group_norm_noalloc", skip, bias)
    if beta.dtype != gamma.dtype:
        raise TypeError("gamma and beta must share one dtype (M)")
    dev = _device_of(X, gamma, beta, skip, bias, Y, S)
    T, M = _code(X, "skip_group_norm_noalloc"), _code(gamma, "skip_group_norm_noalloc gamma")
    with torch.cuda.device(dev):
        check(lib().skip_group_norm_noalloc(T, M, N, C, H, W, _ptr(X), _ptr(gamma), _ptr(beta),
                                            _ptr(skip), bcast, _ptr(bias), float(epsilon),
                                            int(groups), 1 if channels_last else 0, int(activation),
                                            _ptr(Y), _ptr(S), _stream(dev)))
    return SkipGroupNormOutputs(Y, S)


@contextlib.contextmanager
def force_route(route: str):
    """Force "auto", "scalar", "vector", "block", "split" or "flat" routes
    inside the ``with`` block (codes 0-5 of skipnorm_force_route in
    include/skipnorm.h)."""
    code = {"auto": 0, "scalar": 1, "vector": 2, "block": 3, "split": 4, "flat": 5}[route]
    prev = lib().skipnorm_force_route(code)
    try:
        yield
    finally:
        lib().skipnorm_force_route(prev)


@contextlib.contextmanager
def exchange_timeout_us(microseconds: int):
    """Bounded wait of SkipGroupNorm's cluster route inside the ``with``
    block (0 makes every workgroup recompute the other slices itself)."""
    prev = lib().skipnorm_set_exchange_timeout_us(int(microseconds))
    try:
        yield
    finally:
        lib().skipnorm_set_exchange_timeout_us(prev)


def last_route() -> str:
    """Kernel family the calling thread's last successful op call used."""
    return lib().skipnorm_last_route().decode()


def abi_version() -> int:
    return lib().skipnorm_abi_version()


def copy_(dst: torch.Tensor, src: torch.Tensor) -> torch.Tensor:
    """dst <- src with the library's 16-byte copy kernel (measurement aid)."""
    if dst.numel() * dst.element_size() != src.numel() * src.element_size():
        raise ValueError("copy_: byte sizes differ")
    dev = _device_of(dst, src)
    with torch.cuda.device(dev):
        check(lib().skipnorm_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                                  _stream(dev)))
    return dst
