"""Comparison rules between the HIP path and the oracle.

- S (the residual sum) and every value that is exact by construction:
  bitwise equality of the bit patterns (-0 differs from +0).
- float32 outputs and statistics: |gpu - ref| <= 1e-5 * max(1, |ref|)
  (absolute or relative error at most 1e-5).
- float16 outputs: |gpu - ref| <= 2e-3 * |ref| + 2^-14 (about 2 binary16 ulp
  relative, with an absolute floor at the smallest normal binary16 for
  results that cancel to near zero).
- NaN positions must agree; infinities must agree exactly.
"""
from __future__ import annotations

import numpy as np
import torch

F16_REL, F16_ABS = 2e-3, 2.0 ** -14
F32_TOL = 1e-5


def desc(t, shape=None):
    """The C ABI's tensor descriptor for a torch tensor (None for None), with
    the tensor's own shape or the given one (same element count)."""
    if t is None:
        return None
    from group_normalization_amd._lib import SN_F16, SN_F32, tensor_desc
    shape = tuple(t.shape) if shape is None else tuple(shape)
    assert int(np.prod(shape)) == t.numel()
    return tensor_desc(t.data_ptr(), {torch.float32: SN_F32, torch.float16: SN_F16}[t.dtype], shape)


def to_dev(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t):
    return None if t is None else t.detach().cpu().numpy()


def assert_bitwise(got, ref, what):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.dtype == ref.dtype and got.shape == ref.shape, \
        f"{what}: {got.dtype}{got.shape} vs {ref.dtype}{ref.shape}"
    g = got.view(np.uint8).reshape(got.size, -1) if got.size else got
    r = ref.view(np.uint8).reshape(ref.size, -1) if ref.size else ref
    bad = np.nonzero(np.any(g != r, axis=-1))[0] if got.size else []
    assert len(bad) == 0, (f"{what}: {len(bad)} of {got.size} elements differ bitwise; first at "
                           f"{np.unravel_index(bad[0], got.shape)}: {got.ravel()[bad[0]]!r} vs "
                           f"{ref.ravel()[bad[0]]!r}")


def assert_bitwise_nan(got, ref, what):
    """assert_bitwise where NaN positions must agree but NaN payloads (and
    signs) are not compared: inf - inf and 0 * inf give the host's and the
    GPU's own default NaN."""
    got, ref = np.asarray(got), np.asarray(ref)
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({gn.sum()} vs {rn.sum()})"
    assert_bitwise(got[~gn], ref[~rn], what)


def assert_close(got, ref, what):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.dtype == ref.dtype and got.shape == ref.shape, \
        f"{what}: {got.dtype}{got.shape} vs {ref.dtype}{ref.shape}"
    g, r = got.astype(np.float64).ravel(), ref.astype(np.float64).ravel()
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({gn.sum()} vs {rn.sum()})"
    gi, ri = np.isinf(g), np.isinf(r)
    assert np.array_equal(gi, ri) and np.array_equal(g[gi], r[ri]), f"{what}: infinities differ"
    fin = ~(rn | ri)
    g, r = g[fin], r[fin]
    if got.dtype == np.float16:
        tol = F16_REL * np.abs(r) + F16_ABS
    else:
        tol = F32_TOL * np.maximum(1.0, np.abs(r))
    err = np.abs(g - r)
    bad = np.nonzero(err > tol)[0]
    if bad.size:
        i = bad[np.argmax(err[bad] - tol[bad])]
        raise AssertionError(
            f"{what}: {bad.size} of {g.size} outside tolerance; worst gpu={g[i]!r} ref={r[i]!r} "
            f"abs={err[i]:.3g} rel={err[i] / max(abs(r[i]), 1e-300):.3g}")


def report(got, ref):
    """max abs / max rel error (finite elements), for logs."""
    g, r = np.asarray(got, np.float64).ravel(), np.asarray(ref, np.float64).ravel()
    fin = np.isfinite(r) & np.isfinite(g)
    if not fin.any():
        return {"max_abs": 0.0, "max_rel": 0.0}
    e = np.abs(g[fin] - r[fin])
    return {"max_abs": float(e.max()), "max_rel": float((e / np.maximum(np.abs(r[fin]), 1e-30)).max())}
