"""Seeded synthetic inputs for the five reference workloads.

This module draws random tensors and nothing else: it holds none of the
operators' arithmetic, and both the tests (for the oracle and the HIP path)
and the benchmark take their inputs from it.

Recipe (every workload): a fresh ``numpy.random.default_rng(seed)`` (PCG64,
seed 0 by default); tensors drawn in the order listed; distributions

- ``normal``   N(0, 1):   ``rng.standard_normal(shape, dtype=float32)``
- ``normal01`` N(0, 0.1): ``0.1 * rng.standard_normal(shape, dtype=float32)``
- ``uniform``  U(0.5, 1.5): ``rng.uniform(0.5, 1.5, shape)`` (float64)

then one cast (round to nearest even) to the tensor's dtype.  Values are
i.i.d. with no sparsity or outliers; N(0, 1) float16 tensors contain about
5e-5 subnormal values, which exercise the residual-sum rounding.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

F32, F16 = np.float32, np.float16


@dataclass(frozen=True)
class Tensor:
    name: str
    shape: Tuple[int, ...]
    dist: str
    dtype: type


@dataclass(frozen=True)
class Workload:
    name: str
    op: str                      # skip_rms_norm | gated_rms_norm | skip_group_norm
    tensors: Tuple[Tensor, ...]  # in draw order
    attrs: Dict[str, object] = field(default_factory=dict)
    outputs: Tuple[str, ...] = ()

    def tensor(self, name: str) -> Optional[Tensor]:
        for t in self.tensors:
            if t.name == name:
                return t
        return None


def _draw(rng: np.random.Generator, t: Tensor) -> np.ndarray:
    if t.dist == "normal":
        v = rng.standard_normal(t.shape, dtype=np.float32)
    elif t.dist == "normal01":
        v = 0.1 * rng.standard_normal(t.shape, dtype=np.float32)
    elif t.dist == "uniform":
        v = rng.uniform(0.5, 1.5, t.shape)
    else:
        raise ValueError(f"unknown distribution {t.dist!r}")
    return v.astype(t.dtype)


def generate(w: Workload, seed: int = 0) -> Dict[str, np.ndarray]:
    """Host arrays for every input tensor of ``w``, drawn in order."""
    rng = np.random.default_rng(seed)
    return {t.name: _draw(rng, t) for t in w.tensors}


def generate_on_device(w: Workload, seed: int, torch):
    """Device tensors for every input of ``w``, for shapes too large to draw
    on the host in reasonable time (benchmark shapes of 2^27 elements): a
    ``torch.Generator(device="cuda")`` seeded with ``seed``, the tensors
    drawn in order with the same distributions (``torch.randn`` in float32,
    scaled by 0.1 for ``normal01``; ``torch.rand`` mapped to [0.5, 1.5) for
    ``uniform``), then one cast to the tensor's dtype.  The values differ
    from ``generate``'s; they are not compared with the oracle."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = {}
    for t in w.tensors:
        if t.dist in ("normal", "normal01"):
            v = torch.randn(t.shape, generator=g, device="cuda", dtype=torch.float32)
            if t.dist == "normal01":
                v = v * 0.1
        elif t.dist == "uniform":
            v = torch.rand(t.shape, generator=g, device="cuda", dtype=torch.float32) + 0.5
        else:
            raise ValueError(f"unknown distribution {t.dist!r}")
        out[t.name] = v.to({np.float16: torch.float16, np.float32: torch.float32}[t.dtype])
    return out


# ------------------------------------------------------------------ builders
def ssln(name, shape, dtype, bias: bool, epsilon, outputs=("output",)) -> Workload:
    hidden = shape[-1]
    ts = [Tensor("input", shape, "normal", dtype), Tensor("skip", shape, "normal", dtype),
          Tensor("gamma", (hidden,), "uniform", dtype)]
    if bias:
        ts.append(Tensor("bias", (hidden,), "normal01", dtype))
    return Workload(name, "skip_rms_norm", tuple(ts), {"epsilon": epsilon}, tuple(outputs))


def sln(name, shape, dtype, beta: bool, bias: bool, epsilon, outputs=("output",)) -> Workload:
    """Skip layer normalization with the mean removed (non-simplified form)."""
    hidden = shape[-1]
    ts = [Tensor("input", shape, "normal", dtype), Tensor("skip", shape, "normal", dtype),
          Tensor("gamma", (hidden,), "uniform", dtype)]
    if beta:
        ts.append(Tensor("beta", (hidden,), "normal01", dtype))
    if bias:
        ts.append(Tensor("bias", (hidden,), "normal01", dtype))
    return Workload(name, "skip_layer_norm", tuple(ts), {"epsilon": epsilon}, tuple(outputs))


def gated(name, shape, span, dtype, epsilon) -> Workload:
    ts = (Tensor("X", shape, "normal", dtype), Tensor("gate", shape, "normal", dtype),
          Tensor("scale", (span,), "uniform", dtype))
    return Workload(name, "gated_rms_norm", ts, {"epsilon": epsilon}, ("Y",))


def sgn(name, N, C, H, W, dtype, param_dtype, *, channels_last, broadcast_skip, bias, groups,
        activation, epsilon, outputs=("Y",)) -> Workload:
    xshape = (N, H, W, C) if channels_last else (N, C, H, W)
    ts = [Tensor("X", xshape, "normal", dtype),
          Tensor("skip", (N, C) if broadcast_skip else xshape, "normal", dtype)]
    if bias:
        ts.append(Tensor("bias", (C,), "normal01", dtype))
    ts += [Tensor("gamma", (C,), "uniform", param_dtype), Tensor("beta", (C,), "normal01", param_dtype)]
    attrs = {"groups": groups, "activation": activation, "epsilon": epsilon,
             "channels_last": 1 if channels_last else 0}
    return Workload(name, "skip_group_norm", tuple(ts), attrs, tuple(outputs))


# ------------------------------------------------------------------ the five workloads
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    ssln("ssln_f32_64x768", (64, 768), F32, bias=True, epsilon=9.999999960041972e-13,
         outputs=("output", "inv_std_var", "input_skip_bias_sum")),
    ssln("ssln_f16_16x2048x4096", (16, 2048, 4096), F16, bias=False, epsilon=1e-6,
         outputs=("output", "input_skip_bias_sum")),
    gated("gated_f16_8x4096x4096_c128", (8, 4096, 32 * 128), 128, F16, epsilon=1e-5),
    sgn("sgn_f16_nhwc_2x64x64x320", 2, 320, 64, 64, F16, F32, channels_last=True,
        broadcast_skip=False, bias=True, groups=32, activation=1, epsilon=1e-5,
        outputs=("Y", "S")),
    sgn("sgn_f32_nchw_4x1280x32x32", 4, 1280, 32, 32, F32, F16, channels_last=False,
        broadcast_skip=True, bias=False, groups=32, activation=0, epsilon=1e-5),
]}

ORDER: List[str] = list(WORKLOADS)

# Beyond the five: the non-simplified skip layer normalization at the large
# SSLN workload's shape (rows of 4096 float16, S requested), with beta.
EXTRA_WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    sln("sln_f16_16x2048x4096", (16, 2048, 4096), F16, beta=True, bias=False, epsilon=1e-5,
        outputs=("output", "input_skip_bias_sum")),
]}


def io_bytes(w: Workload) -> int:
    """Algorithmic bytes of one op call: every input read once plus every
    requested output written once."""
    total = 0
    for t in w.tensors:
        total += int(np.prod(t.shape)) * np.dtype(t.dtype).itemsize
    first = w.tensors[0]
    data = int(np.prod(first.shape)) * np.dtype(first.dtype).itemsize
    for o in w.outputs:
        if o in ("mean", "inv_std_var"):
            total += int(np.prod(first.shape[:-1])) * 4
        else:
            total += data
    return total
