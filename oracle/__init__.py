"""CPU oracle for the fused skip-add + normalize operators.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the product package never imports
it.  The arithmetic lives in ``skipnorm_oracle.c`` (plain C99, single thread,
float64 statistics); this module only moves numpy arrays in and out of it.

Functions take and return host numpy arrays.  float16 tensors are passed as
``numpy.float16`` arrays (their bit patterns are what the C code reads).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "skipnorm_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

#: The flags that make every float operation in the C source a single IEEE
#: operation in the precision written (no contraction, no fast-math).
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle source with gcc into a shared library."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-I", _HERE, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _type_code(dtype) -> int:
    dtype = np.dtype(dtype)
    if dtype == np.float32:
        return 0
    if dtype == np.float16:
        return 1
    raise TypeError(f"oracle supports float32 and float16, not {dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _host(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


class Oracle:
    """One loaded build of the oracle library (the default one, or a build
    of a deliberately altered source used by the planted-mistake tests)."""

    def __init__(self, lib_path: str = LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_f16_to_f32_array.argtypes = [vp, vp, i64]
        lib.oracle_f16_to_f32_array.restype = None
        lib.oracle_f32_to_f16_array.argtypes = [vp, vp, i64]
        lib.oracle_f32_to_f16_array.restype = None
        lib.oracle_skip_rms_norm.argtypes = [ci, i64, i64, vp, vp, vp, vp, f32,
                                             vp, vp, vp, vp]
        lib.oracle_skip_rms_norm.restype = ci
        lib.oracle_skip_layer_norm.argtypes = [ci, i64, i64, vp, vp, vp, vp, vp, f32,
                                               vp, vp, vp, vp]
        lib.oracle_skip_layer_norm.restype = ci
        lib.oracle_gated_rms_norm.argtypes = [ci, i64, i64, vp, vp, vp, f32, vp]
        lib.oracle_gated_rms_norm.restype = ci
        lib.oracle_skip_group_norm.argtypes = [ci, ci, i64, i64, i64, i64, ci,
                                               vp, vp, vp, vp, ci, vp, f32, i64,
                                               ci, vp, vp]
        lib.oracle_skip_group_norm.restype = ci
        self.lib = lib
        self.path = lib_path

    # -------------------------------------------------------------- convert
    def f16_bits_to_f32(self, bits):
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float32)
        self.lib.oracle_f16_to_f32_array(_ptr(bits), _ptr(out), bits.size)
        return out

    def f32_to_f16_bits(self, values):
        values = np.ascontiguousarray(values, dtype=np.float32)
        out = np.empty(values.shape, np.uint16)
        self.lib.oracle_f32_to_f16_array(_ptr(values), _ptr(out), values.size)
        return out

    def f64_to_f16_bits(self, value: float) -> int:
        return int(self.lib.oracle_f64_to_f16(float(value)))

    # -------------------------------------------------------------- ops
    def skip_rms_norm(self, input, skip, gamma, bias=None,
                      epsilon=9.999999960041972e-13, *, want_mean=False,
                      want_inv_std_var=False, want_sum=False):
        """SkipSimplifiedLayerNormalization over the last axis.

        Returns (output, mean, inv_std_var, input_skip_bias_sum); entries not
        requested are None.  mean/inv_std_var have the input's shape with the
        last axis replaced by 1 (float32).
        """
        input = _host(input)
        T = _type_code(input.dtype)
        skip = _host(skip, input.dtype)
        gamma = _host(gamma, input.dtype)
        bias = _host(bias, input.dtype)
        hidden = input.shape[-1]
        rows = input.size // hidden if hidden else 0
        stat_shape = input.shape[:-1] + (1,)
        out = np.empty_like(input)
        mean = np.empty(stat_shape, np.float32) if want_mean else None
        inv = np.empty(stat_shape, np.float32) if want_inv_std_var else None
        s = np.empty_like(input) if want_sum else None
        rc = self.lib.oracle_skip_rms_norm(T, rows, hidden, _ptr(input), _ptr(skip),
                                           _ptr(gamma), _ptr(bias), float(epsilon),
                                           _ptr(out), _ptr(mean), _ptr(inv), _ptr(s))
        if rc != 0:
            raise ValueError(f"oracle_skip_rms_norm rejected its arguments ({rc})")
        return out, mean, inv, s

    def skip_layer_norm(self, input, skip, gamma, beta=None, bias=None,
                        epsilon=9.999999960041972e-13, *, want_mean=False,
                        want_inv_std_var=False, want_sum=False):
        """Skip layer normalization with the mean removed, over the last axis.

        Returns (output, mean, inv_std_var, input_skip_bias_sum) like
        skip_rms_norm; here mean is the row mean and inv_std_var the inverse
        standard deviation.
        """
        input = _host(input)
        T = _type_code(input.dtype)
        skip = _host(skip, input.dtype)
        gamma = _host(gamma, input.dtype)
        beta = _host(beta, input.dtype)
        bias = _host(bias, input.dtype)
        hidden = input.shape[-1]
        rows = input.size // hidden if hidden else 0
        stat_shape = input.shape[:-1] + (1,)
        out = np.empty_like(input)
        mean = np.empty(stat_shape, np.float32) if want_mean else None
        inv = np.empty(stat_shape, np.float32) if want_inv_std_var else None
        s = np.empty_like(input) if want_sum else None
        rc = self.lib.oracle_skip_layer_norm(T, rows, hidden, _ptr(input), _ptr(skip),
                                             _ptr(gamma), _ptr(beta), _ptr(bias), float(epsilon),
                                             _ptr(out), _ptr(mean), _ptr(inv), _ptr(s))
        if rc != 0:
            raise ValueError(f"oracle_skip_layer_norm rejected its arguments ({rc})")
        return out, mean, inv, s

    def gated_rms_norm(self, X, scale, gate, epsilon=1e-5):
        """GatedRMSNorm with span C = scale.size over flat rows of X."""
        X = _host(X)
        T = _type_code(X.dtype)
        scale = _host(scale, X.dtype)
        gate = _host(gate, X.dtype)
        Y = np.empty_like(X)
        rc = self.lib.oracle_gated_rms_norm(T, X.size, scale.size, _ptr(X), _ptr(scale),
                                            _ptr(gate), float(epsilon), _ptr(Y))
        if rc != 0:
            raise ValueError(f"oracle_gated_rms_norm rejected its arguments ({rc})")
        return Y

    def skip_group_norm(self, X, gamma, beta, skip, bias=None, *, groups, activation,
                        epsilon=1e-5, channels_last=1, want_sum=False):
        """SkipGroupNorm; X is (N,H,W,C) when channels_last else (N,C,H,W).

        ``skip`` is either X's shape (full) or (N,C)/(N,1,1,C) (broadcast).
        Returns (Y, S); S is None unless want_sum.
        """
        X = _host(X)
        T = _type_code(X.dtype)
        gamma = _host(gamma)
        M = _type_code(gamma.dtype)
        beta = _host(beta, gamma.dtype)
        skip = _host(skip, X.dtype)
        bias = _host(bias, X.dtype)
        if X.ndim != 4:
            raise ValueError("X must be rank 4")
        if channels_last:
            N, H, W, C = X.shape
        else:
            N, C, H, W = X.shape
        if skip.shape == X.shape:
            bcast = 0
        elif skip.shape in ((N, C), (N, 1, 1, C)):
            bcast = 1
        else:
            raise ValueError(f"skip shape {skip.shape} matches neither X nor (N, C)")
        Y = np.empty_like(X)
        S = np.empty_like(X) if want_sum else None
        rc = self.lib.oracle_skip_group_norm(T, M, N, C, H, W, 1 if channels_last else 0,
                                             _ptr(X), _ptr(gamma), _ptr(beta), _ptr(skip),
                                             bcast, _ptr(bias), float(epsilon), int(groups),
                                             int(activation), _ptr(Y), _ptr(S))
        if rc != 0:
            raise ValueError(f"oracle_skip_group_norm rejected its arguments ({rc})")
        return Y, S


_default = None


def default() -> Oracle:
    """The oracle built from the committed source (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def f16_bits_to_f32(bits):
    return default().f16_bits_to_f32(bits)


def f32_to_f16_bits(values):
    return default().f32_to_f16_bits(values)


def f64_to_f16_bits(value):
    return default().f64_to_f16_bits(value)


def skip_rms_norm(*args, **kwargs):
    return default().skip_rms_norm(*args, **kwargs)


def skip_layer_norm(*args, **kwargs):
    return default().skip_layer_norm(*args, **kwargs)


def gated_rms_norm(*args, **kwargs):
    return default().gated_rms_norm(*args, **kwargs)


def skip_group_norm(*args, **kwargs):
    return default().skip_group_norm(*args, **kwargs)
