"""Fused skip-add + normalize operators on AMD Instinct MI355X (gfx950).

Python binding of libskipnorm (C ABI in ``include/skipnorm.h``): argument
marshalling only.  Tensors are torch tensors on a ROCm device, passed as the
ABI's tensor descriptors (data pointer, dtype, rank, shape); torch provides
device memory and the current stream; the library validates every shape,
dtype and attribute, and every step of the computation runs in its HIP
kernels.  Outputs are allocated here with the shapes and dtypes the operator
contracts define.

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

from ._lib import SN_BF16, SN_F16, SN_F32, SkipNormError, check, lib, tensor_desc

__all__ = ["skip_layer_norm", "skip_rms_norm", "gated_rms_norm", "skip_group_norm", "skip_group_norm_workspace_size",
           "skip_group_norm_noalloc",
           "SkipRmsNormOutputs", "SkipGroupNormOutputs", "SkipNormError", "force_route",
           "last_route", "exchange_timeout_us", "abi_version", "copy_"]

#: Attribute defaults from the pages' Attributes tables.
SSLN_EPSILON = 9.999999960041972e-13
GATED_EPSILON = 1e-5
SGN_EPSILON = 1e-5

_DTYPES = {torch.float32: SN_F32, torch.float16: SN_F16, torch.bfloat16: SN_BF16}
_UNKNOWN_DTYPE = -1  # rejected by the library with SN_ERR_DTYPE


class SkipRmsNormOutputs(NamedTuple):
    output: torch.Tensor
    mean: Optional[torch.Tensor]
    inv_std_var: Optional[torch.Tensor]
    input_skip_bias_sum: Optional[torch.Tensor]


class SkipGroupNormOutputs(NamedTuple):
    Y: torch.Tensor
    S: Optional[torch.Tensor]


def _desc(t: Optional[torch.Tensor]):
    """The tensor's sn_tensor descriptor (None for an absent tensor)."""
    if t is None:
        return None
    return tensor_desc(t.data_ptr(), _DTYPES.get(t.dtype, _UNKNOWN_DTYPE), t.shape)


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


def _stat_shape(input: torch.Tensor):
    return tuple(input.shape[:-1]) + (1,) if input.dim() >= 1 else (1,)


def skip_rms_norm(input: torch.Tensor, skip: torch.Tensor, gamma: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, epsilon: float = SSLN_EPSILON, *,
                  want_mean: bool = False, want_inv_std_var: bool = False,
                  want_sum: bool = False) -> SkipRmsNormOutputs:
    """SkipSimplifiedLayerNormalization over the last axis.

    input/skip: (token_count, hidden) or (batch, sequence, hidden), type T;
    gamma, bias: (hidden,).  Returns (output, mean, inv_std_var,
    input_skip_bias_sum); optional entries are None unless requested.
    """
    dev = _device_of(input, skip, gamma, bias)
    output = torch.empty_like(input)
    mean = torch.empty(_stat_shape(input), dtype=torch.float32, device=dev) if want_mean else None
    inv = torch.empty(_stat_shape(input), dtype=torch.float32, device=dev) if want_inv_std_var else None
    s = torch.empty_like(input) if want_sum else None
    with torch.cuda.device(dev):
        check(lib().skip_rms_norm(_desc(input), _desc(skip), _desc(gamma), _desc(bias),
                                  float(epsilon), _desc(output), _desc(mean), _desc(inv), _desc(s),
                                  _stream(dev)))
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
    dev = _device_of(input, skip, gamma, beta, bias)
    output = torch.empty_like(input)
    mean = torch.empty(_stat_shape(input), dtype=torch.float32, device=dev) if want_mean else None
    inv = torch.empty(_stat_shape(input), dtype=torch.float32, device=dev) if want_inv_std_var else None
    s = torch.empty_like(input) if want_sum else None
    with torch.cuda.device(dev):
        check(lib().skip_layer_norm(_desc(input), _desc(skip), _desc(gamma), _desc(beta),
                                    _desc(bias), float(epsilon), _desc(output), _desc(mean),
                                    _desc(inv), _desc(s), _stream(dev)))
    return SkipRmsNormOutputs(output, mean, inv, s)


def gated_rms_norm(X: torch.Tensor, scale: torch.Tensor, gate: torch.Tensor,
                   epsilon: float = GATED_EPSILON) -> torch.Tensor:
    """GatedRMSNorm: RMS over each contiguous run of C = scale.numel()
    elements of X (rows counted flat), times scale and SiLU(gate).  scale may
    be spelled (C), (1, C) or (C, 1)."""
    dev = _device_of(X, scale, gate)
    Y = torch.empty_like(X)
    with torch.cuda.device(dev):
        check(lib().gated_rms_norm(_desc(X), _desc(scale), _desc(gate), float(epsilon), _desc(Y),
                                   _stream(dev)))
    return Y


def skip_group_norm_workspace_size(X: torch.Tensor, groups: int, channels_last: int = 1) -> int:
    """Workspace bytes skip_group_norm needs for X (only its shape and dtype
    are read)."""
    out = ctypes.c_size_t(0)
    check(lib().skip_group_norm_workspace_size(_desc(X), int(groups), 1 if channels_last else 0,
                                               ctypes.byref(out)))
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
    dev = _device_of(X, gamma, beta, skip, bias)
    Y = torch.empty_like(X)
    S = torch.empty_like(X) if want_sum else None
    if workspace is None:
        need = skip_group_norm_workspace_size(X, groups, channels_last)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev:
        raise ValueError("workspace must be on the tensors' device")
    with torch.cuda.device(dev):
        check(lib().skip_group_norm(_desc(X), _desc(gamma), _desc(beta), _desc(skip), _desc(bias),
                                    float(epsilon), int(groups), 1 if channels_last else 0,
                                    int(activation), _desc(Y), _desc(S),
                                    ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(), _stream(dev)))
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
    dev = _device_of(X, gamma, beta, skip, bias, Y, S)
    with torch.cuda.device(dev):
        check(lib().skip_group_norm_noalloc(_desc(X), _desc(gamma), _desc(beta), _desc(skip),
                                            _desc(bias), float(epsilon), int(groups),
                                            1 if channels_last else 0, int(activation), _desc(Y),
                                            _desc(S), _stream(dev)))
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
        check(lib().skipnorm_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                  src.numel() * src.element_size(), _stream(dev)))
    return dst
