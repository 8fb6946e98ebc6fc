"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises
``AssertionError`` when the oracle disagrees with:

- the hand-worked closed forms in ``tests/golden/hand_cases.json``;
- numpy's IEEE-754 binary16 conversions (a library routine);
- the float64 CPU library routines the operators reduce to in special cases
  (``torch.nn.functional.rms_norm``, ``group_norm``, ``instance_norm``,
  ``layer_norm``, ``silu``);
- invariants that the operator definitions imply (scale invariance, zero
  gate, broadcast equals expanded skip, layout permutation, S request not
  changing Y, ...).

The same functions run against the committed oracle (``test_oracle_pins``)
and against deliberately altered builds of it (``test_oracle_mutants``), which
must each fail at least one pin.
"""
from __future__ import annotations

import json
import os
from decimal import Decimal

import numpy as np
import torch
import torch.nn.functional as F

from closed_form import evaluate, round_to

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")
EPS_SSLN = 9.999999960041972e-13


def load_hand_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


# ----------------------------------------------------------------- helpers
def ulp_diff(a, b):
    """Distance in units in the last place between same-dtype float arrays
    (NaN positions must agree; they count as 0)."""
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.dtype == b.dtype and a.shape == b.shape
    na, nb = np.isnan(a), np.isnan(b)
    assert np.array_equal(na, nb), "NaN positions differ"
    itype = np.int16 if a.dtype == np.float16 else np.int32
    wide = np.int64

    def ordered(x):
        i = x.view(itype).astype(wide)
        sign_bit = np.array(1, wide) << (8 * x.dtype.itemsize - 1)
        return np.where(i < 0, -(i + sign_bit), i)  # -0 and +0 map to 0

    d = np.abs(ordered(a) - ordered(b))
    d[na] = 0
    return d


def assert_within_ulp(got, ref, max_ulp, what):
    d = ulp_diff(got, ref)
    worst = int(d.max()) if d.size else 0
    assert worst <= max_ulp, f"{what}: {worst} ulp apart (allowed {max_ulp})"


def residual_sum_numpy(x, skip, bias, dtype):
    """S by numpy's own float32 additions and dtype rounding (library ops)."""
    s = x.astype(np.float32) + skip.astype(np.float32)
    if bias is not None:
        s = s + bias.astype(np.float32)
    return s.astype(dtype)


# ----------------------------------------------------------------- hand cases
def _expect_array(exprs, eps, dtype):
    flat = np.array(exprs, dtype=object)
    out = np.empty(flat.shape, dtype=dtype)
    for idx, e in np.ndenumerate(flat):
        out[idx] = round_to(evaluate(e, eps), dtype)
    return out


def _bits(hexes):
    return np.array(np.vectorize(lambda h: int(h, 16))(np.array(hexes, dtype=object)),
                    dtype=np.uint16)


def run_hand_case(orc, case):
    dt = np.dtype(case["dtype"])
    eps32 = np.float32(case["epsilon"])
    eps = Decimal(float(eps32))
    arr = lambda v, d=dt: None if v is None else np.array(v, dtype=d)
    if case["op"] == "skip_rms_norm":
        out, mean, inv, s = orc.skip_rms_norm(
            arr(case["input"]), arr(case["skip"]), arr(case["gamma"]), arr(case["bias"]),
            float(eps32), want_mean=True, want_inv_std_var=True, want_sum=True)
        got = {"output": out, "mean": mean, "inv_std_var": inv, "input_skip_bias_sum": s}
    elif case["op"] == "skip_layer_norm":
        out, mean, inv, s = orc.skip_layer_norm(
            arr(case["input"]), arr(case["skip"]), arr(case["gamma"]), arr(case["beta"]),
            arr(case["bias"]), float(eps32), want_mean=True, want_inv_std_var=True, want_sum=True)
        got = {"output": out, "mean": mean, "inv_std_var": inv, "input_skip_bias_sum": s}
    elif case["op"] == "gated_rms_norm":
        got = {"Y": orc.gated_rms_norm(arr(case["X"]), arr(case["scale"]), arr(case["gate"]),
                                       float(eps32))}
    elif case["op"] == "skip_group_norm":
        pdt = np.dtype(case["param_dtype"])
        Y, S = orc.skip_group_norm(arr(case["X"]), arr(case["gamma"], pdt), arr(case["beta"], pdt),
                                   arr(case["skip"]), arr(case["bias"]), groups=case["groups"],
                                   activation=case["activation"], epsilon=float(eps32),
                                   channels_last=case["channels_last"], want_sum=True)
        got = {"Y": Y, "S": S}
    else:
        raise AssertionError(case["op"])
    for name, exprs in case["expect"].items():
        if name.endswith("_bits"):
            g = got[name[:-5]]
            want = _bits(exprs)
            assert np.array_equal(g.view(np.uint16), want), \
                f"{case['id']} {name}: {g.view(np.uint16)} != {want}"
        else:
            g = got[name]
            want = _expect_array(exprs, eps, g.dtype)
            assert np.array_equal(g, want), f"{case['id']} {name}: {g} != {want}"


def pin_hand_cases(orc):
    for case in load_hand_cases():
        run_hand_case(orc, case)


# ----------------------------------------------------------------- binary16
def pin_f16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = orc.f16_bits_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])


def f32_patterns_structured():
    """Every sign/exponent/top-10-fraction combination of binary32 (2^19),
    each with the low 13 fraction bits set to the values that decide binary16
    rounding: exact, just above zero, just below/at/above the half, all ones.
    Below 2^-14 those low bits still matter, so the subnormal band of binary16
    (binary32 exponents 102..112) additionally gets a dense random sample."""
    hi = np.arange(1 << 19, dtype=np.uint32) << np.uint32(13)
    lows = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x0800, 0x17FF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(1234)
    sub = rng.integers(0, 1 << 23, size=1 << 20, dtype=np.uint32)
    exps = rng.integers(102, 113, size=1 << 20, dtype=np.uint32) << np.uint32(23)
    signs = rng.integers(0, 2, size=1 << 20, dtype=np.uint32) << np.uint32(31)
    return np.concatenate([pats, sub | exps | signs])


def pin_f32_to_f16_structured(orc):
    pats = f32_patterns_structured()
    vals = pats.view(np.float32)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = orc.f32_to_f16_bits(vals)
    keep = ~np.isnan(vals)
    bad = np.nonzero((got != ref) & keep)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {hex(int(pats[bad[0]]))}"
    assert np.all(np.isnan(orc.f16_bits_to_f32(got[~keep])))


def pin_f64_to_f16_ties(orc):
    cases = {
        1 + 2.0 ** -11: 0x3C00,                  # tie -> even (1.0)
        1 + 3 * 2.0 ** -11: 0x3C02,              # tie -> even (1 + 2^-9)
        1 + 2.0 ** -11 + 2.0 ** -40: 0x3C01,     # just above the tie
        65504.0: 0x7BFF,
        65519.99: 0x7BFF,
        65520.0: 0x7C00,                         # overflow midpoint -> inf
        2.0 ** -25: 0x0000,                      # tie between 0 and 2^-24 -> 0
        3 * 2.0 ** -25: 0x0002,                  # tie between 1 and 2 quanta -> 2
        -(2.0 ** -25): 0x8000,
        2.0 ** -14: 0x0400,                      # smallest normal
        2.0 ** -14 - 2.0 ** -25: 0x0400,         # rounds up across the boundary
        -2.0: 0xC000,
        0.1: 0x2E66,
    }
    for v, want in cases.items():
        got = orc.f64_to_f16_bits(v)
        assert got == want, f"f64->f16({v!r}) = {hex(got)}, want {hex(want)}"


# ----------------------------------------------------------------- SSLN
def pin_ssln_matches_torch(orc):
    rng = np.random.default_rng(11)
    for dt, rows, hidden, with_bias in [(np.float32, 8, 768, True), (np.float32, 5, 33, False),
                                        (np.float16, 6, 256, True), (np.float16, 3, 17, False)]:
        x = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        k = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        g = rng.uniform(0.5, 1.5, hidden).astype(dt)
        b = (0.1 * rng.standard_normal(hidden, dtype=np.float32)).astype(dt) if with_bias else None
        eps = 1e-6
        out, _, inv, s = orc.skip_rms_norm(x, k, g, b, eps, want_inv_std_var=True, want_sum=True)
        s_ref = residual_sum_numpy(x, k, b, dt)
        assert np.array_equal(s.view(np.uint8), s_ref.view(np.uint8)), "S differs from numpy's sum"
        st = torch.from_numpy(s_ref.astype(np.float64))
        y = F.rms_norm(st, (hidden,), torch.from_numpy(g.astype(np.float64)), eps=float(np.float32(eps)))
        assert_within_ulp(out, y.numpy().astype(dt), 1, f"SSLN {np.dtype(dt)} output vs rms_norm")
        inv_ref = torch.rsqrt(st.pow(2).mean(-1, keepdim=True) + float(np.float32(eps)))
        assert_within_ulp(inv, inv_ref.numpy().astype(np.float32), 1, "SSLN inv_std_var")


def pin_ssln_invariants(orc):
    rng = np.random.default_rng(12)
    for dt in (np.float32, np.float16):
        rows, hidden = 7, 96
        x = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        k = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        b = (0.1 * rng.standard_normal(hidden, dtype=np.float32)).astype(dt)
        ones = np.ones(hidden, dt)
        # gamma = 1: every row of the output has mean square ms/(ms + eps).
        eps = 0.01
        out, _, inv, s = orc.skip_rms_norm(x, k, ones, b, eps, want_inv_std_var=True, want_sum=True)
        ms = (s.astype(np.float64) ** 2).mean(-1)
        msy = (out.astype(np.float64) ** 2).mean(-1)
        tol = 1e-6 if dt == np.float32 else 2e-3
        assert np.allclose(msy, ms / (ms + np.float32(eps)), rtol=tol), "mean square of output"
        # Scale invariance with eps = 0: powers of two scale exactly.
        g = rng.uniform(0.5, 1.5, hidden).astype(dt)
        y1 = orc.skip_rms_norm(x, k, g, b, 0.0)[0]
        y2 = orc.skip_rms_norm((x * dt(4)).astype(dt), (k * dt(4)).astype(dt), g,
                               (b * dt(4)).astype(dt), 0.0)[0]
        assert np.array_equal(y1.view(np.uint8), y2.view(np.uint8)), "scale invariance"
        # Requesting S / statistics does not change the output; mean is zero.
        y3, mean, inv3, _ = orc.skip_rms_norm(x, k, g, b, 1e-6, want_mean=True,
                                              want_inv_std_var=True, want_sum=True)
        y4 = orc.skip_rms_norm(x, k, g, b, 1e-6)[0]
        assert np.array_equal(y3.view(np.uint8), y4.view(np.uint8)), "S request changed Y"
        assert np.all(mean == 0)
        # The statistic sees S rounded to T: feeding S back with a zero skip
        # gives the same output bit for bit.
        z = np.zeros_like(x)
        s = orc.skip_rms_norm(x, k, g, b, 1e-6, want_sum=True)[3]
        y5 = orc.skip_rms_norm(s, z, g, None, 1e-6)[0]
        assert np.array_equal(y4.view(np.uint8), y5.view(np.uint8)), "statistic not on rounded S"


# ----------------------------------------------------------------- SkipLayerNorm
def pin_sln_matches_torch(orc):
    rng = np.random.default_rng(13)
    for dt, rows, hidden, with_beta, with_bias in [(np.float32, 8, 768, True, True),
                                                   (np.float32, 5, 33, False, False),
                                                   (np.float16, 6, 256, True, False),
                                                   (np.float16, 3, 17, False, True)]:
        x = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        k = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        g = rng.uniform(0.5, 1.5, hidden).astype(dt)
        be = (0.1 * rng.standard_normal(hidden, dtype=np.float32)).astype(dt) if with_beta else None
        b = (0.1 * rng.standard_normal(hidden, dtype=np.float32)).astype(dt) if with_bias else None
        eps = 1e-5
        out, mean, inv, s = orc.skip_layer_norm(x, k, g, be, b, eps, want_mean=True,
                                                want_inv_std_var=True, want_sum=True)
        s_ref = residual_sum_numpy(x, k, b, dt)
        assert np.array_equal(s.view(np.uint8), s_ref.view(np.uint8)), "S differs from numpy's sum"
        st = torch.from_numpy(s_ref.astype(np.float64))
        y = F.layer_norm(st, (hidden,), torch.from_numpy(g.astype(np.float64)),
                         None if be is None else torch.from_numpy(be.astype(np.float64)),
                         eps=float(np.float32(eps)))
        assert_within_ulp(out, y.numpy().astype(dt), 1, f"SLN {np.dtype(dt)} output vs layer_norm")
        assert_within_ulp(mean, st.mean(-1, keepdim=True).numpy().astype(np.float32), 1, "SLN mean")
        var = st.var(-1, unbiased=False, keepdim=True)
        assert_within_ulp(inv, torch.rsqrt(var + float(np.float32(eps))).numpy().astype(np.float32), 1,
                          "SLN inv_std_var")


def pin_sln_invariants(orc):
    rng = np.random.default_rng(14)
    for dt in (np.float32, np.float16):
        rows, hidden = 6, 64
        x = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        k = rng.standard_normal((rows, hidden), dtype=np.float32).astype(dt)
        g = rng.uniform(0.5, 1.5, hidden).astype(dt)
        be = (0.1 * rng.standard_normal(hidden, dtype=np.float32)).astype(dt)
        ones, zeros = np.ones(hidden, dt), np.zeros(hidden, dt)
        # gamma = 1, beta = 0: each output row has mean 0 and variance v/(v + eps).
        eps = 0.01
        out, _, _, s = orc.skip_layer_norm(x, k, ones, None, None, eps, want_sum=True)
        v = s.astype(np.float64).var(-1)
        tol = 1e-6 if dt == np.float32 else 2e-3
        assert np.allclose(out.astype(np.float64).mean(-1), 0, atol=tol * 10), "output mean"
        assert np.allclose(out.astype(np.float64).var(-1), v / (v + np.float32(eps)), rtol=tol * 5), "variance"
        # A zero-mean S (values in +- pairs, exact cancellation) makes the
        # operator the simplified one: outputs equal bit for bit.
        half = rng.standard_normal((rows, hidden // 2), dtype=np.float32).astype(dt)
        xs = np.empty((rows, hidden), dt)
        xs[:, 0::2], xs[:, 1::2] = half, -half
        y_ln, m_ln, inv_ln, _ = orc.skip_layer_norm(xs, np.zeros_like(xs), g, None, None, 1e-6,
                                                    want_mean=True, want_inv_std_var=True)
        y_rms, _, inv_rms, _ = orc.skip_rms_norm(xs, np.zeros_like(xs), g, None, 1e-6, want_inv_std_var=True)
        assert np.all(m_ln == 0)
        assert np.array_equal(y_ln.view(np.uint8), y_rms.view(np.uint8)), "zero-mean rows != simplified"
        assert np.array_equal(inv_ln, inv_rms)
        # beta adds after the normalization: beta = 0 equals no beta; a beta
        # of ones shifts every output by exactly one (float32).
        y0 = orc.skip_layer_norm(x, k, g, zeros, None, 1e-5)[0]
        y1 = orc.skip_layer_norm(x, k, g, None, None, 1e-5)[0]
        assert np.array_equal(y0.view(np.uint8), y1.view(np.uint8)), "beta = 0"
        # Scale invariance with eps = 0: powers of two scale exactly.
        y2 = orc.skip_layer_norm(x, k, g, be, None, 0.0)[0]
        y3 = orc.skip_layer_norm((x * dt(4)).astype(dt), (k * dt(4)).astype(dt), g, be, None, 0.0)[0]
        assert np.array_equal(y2.view(np.uint8), y3.view(np.uint8)), "scale invariance"
        # Requesting S / statistics does not change the output.
        y4 = orc.skip_layer_norm(x, k, g, be, None, 1e-5, want_mean=True, want_inv_std_var=True,
                                 want_sum=True)[0]
        y5 = orc.skip_layer_norm(x, k, g, be, None, 1e-5)[0]
        assert np.array_equal(y4.view(np.uint8), y5.view(np.uint8)), "S request changed output"


# ----------------------------------------------------------------- Gated
def _gated_torch(x, scale, gate, eps, dt):
    C = scale.size
    xt = torch.from_numpy(x.astype(np.float64)).reshape(-1, C)
    gt = torch.from_numpy(gate.astype(np.float64)).reshape(-1, C)
    st = torch.from_numpy(scale.astype(np.float64)).reshape(C)
    y = F.rms_norm(xt, (C,), st, eps=float(np.float32(eps))) * F.silu(gt)
    return y.reshape(x.shape).numpy().astype(dt)


def pin_gated_matches_torch(orc):
    rng = np.random.default_rng(21)
    for dt, shape, C in [(np.float32, (4, 6, 64), 32), (np.float16, (3, 256), 128),
                         (np.float16, (5, 3, 10), 5), (np.float32, (7,), 7), (np.float32, (2, 9), 1)]:
        x = rng.standard_normal(shape, dtype=np.float32).astype(dt)
        gate = rng.standard_normal(shape, dtype=np.float32).astype(dt)
        scale = rng.uniform(0.5, 1.5, C).astype(dt)
        eps = 1e-5
        y = orc.gated_rms_norm(x, scale, gate, eps)
        assert_within_ulp(y, _gated_torch(x, scale, gate, eps, dt), 1, f"gated {shape} C={C}")


def pin_gated_invariants(orc):
    rng = np.random.default_rng(22)
    for dt in (np.float32, np.float16):
        x = rng.standard_normal((6, 4 * 16), dtype=np.float32).astype(dt)
        gate = rng.standard_normal((6, 64), dtype=np.float32).astype(dt)
        scale = rng.uniform(0.5, 1.5, 16).astype(dt)
        y = orc.gated_rms_norm(x, scale, gate, 1e-5)
        # gate = 0 gives exactly zero.
        assert np.all(orc.gated_rms_norm(x, scale, np.zeros_like(gate), 1e-5) == 0)
        # Packed (R, H*C) equals (R*H, C) and (R, H, C); scale spellings agree.
        for xs, gs, sc in [(x.reshape(24, 16), gate.reshape(24, 16), scale),
                           (x.reshape(6, 4, 16), gate.reshape(6, 4, 16), scale.reshape(1, 16)),
                           (x.ravel(), gate.ravel(), scale.reshape(16, 1))]:
            y2 = orc.gated_rms_norm(xs, sc, gs, 1e-5)
            assert np.array_equal(y2.reshape(y.shape).view(np.uint8), y.view(np.uint8))
        # Scale invariance in X with eps = 0.
        y0 = orc.gated_rms_norm(x, scale, gate, 0.0)
        y1 = orc.gated_rms_norm((x * dt(8)).astype(dt), scale, gate, 0.0)
        assert np.array_equal(y0.view(np.uint8), y1.view(np.uint8))
        # Large positive gate: SiLU(g) -> g, so Y -> RMSNorm(x) * scale * g.
        big = np.full_like(gate, 30)
        yb = orc.gated_rms_norm(x, scale, big, 0.0)
        xt = torch.from_numpy(x.astype(np.float64)).reshape(-1, 16)
        ref = F.rms_norm(xt, (16,), torch.from_numpy(scale.astype(np.float64)), eps=0.0)
        ref = (ref * 30).reshape(x.shape).numpy()
        tol = 1e-5 if dt == np.float32 else 2e-3
        assert np.allclose(yb.astype(np.float64), ref, rtol=tol, atol=1e-6)


# ----------------------------------------------------------------- SGN
def _sgn_torch(s_nhwc_or_nchw, gamma, beta, groups, eps, act, channels_last, dt):
    s = torch.from_numpy(s_nhwc_or_nchw.astype(np.float64))
    if channels_last:
        s = s.permute(0, 3, 1, 2)
    y = F.group_norm(s, groups, torch.from_numpy(gamma.astype(np.float64)),
                     torch.from_numpy(beta.astype(np.float64)), eps=float(np.float32(eps)))
    if act:
        y = F.silu(y)
    if channels_last:
        y = y.permute(0, 2, 3, 1)
    return np.ascontiguousarray(y.numpy()).astype(dt)


def _sgn_inputs(rng, dt, pdt, N, C, H, W, channels_last, bcast, with_bias):
    shape = (N, H, W, C) if channels_last else (N, C, H, W)
    x = rng.standard_normal(shape, dtype=np.float32).astype(dt)
    skip = rng.standard_normal((N, C) if bcast else shape, dtype=np.float32).astype(dt)
    bias = (0.1 * rng.standard_normal(C, dtype=np.float32)).astype(dt) if with_bias else None
    gamma = rng.uniform(0.5, 1.5, C).astype(pdt)
    beta = (0.1 * rng.standard_normal(C, dtype=np.float32)).astype(pdt)
    return x, skip, bias, gamma, beta


def _expand_skip(skip, N, C, H, W, channels_last):
    if channels_last:
        return np.broadcast_to(skip.reshape(N, 1, 1, C), (N, H, W, C)).copy()
    return np.broadcast_to(skip.reshape(N, C, 1, 1), (N, C, H, W)).copy()


def pin_sgn_matches_torch(orc):
    rng = np.random.default_rng(31)
    combos = [
        (np.float32, np.float32, 2, 12, 5, 3, 1, False, True, 0, 4),
        (np.float16, np.float32, 2, 20, 4, 6, 1, False, True, 1, 2),
        (np.float32, np.float16, 3, 16, 3, 5, 0, True, False, 0, 8),
        (np.float16, np.float16, 2, 8, 7, 2, 0, False, True, 1, 8),
        (np.float16, np.float32, 2, 6, 3, 4, 1, True, True, 1, 3),
    ]
    for dt, pdt, N, C, H, W, cl, bcast, with_bias, act, groups in combos:
        x, skip, bias, gamma, beta = _sgn_inputs(rng, dt, pdt, N, C, H, W, cl, bcast, with_bias)
        Y, S = orc.skip_group_norm(x, gamma, beta, skip, bias, groups=groups, activation=act,
                                   epsilon=1e-5, channels_last=cl, want_sum=True)
        full = _expand_skip(skip, N, C, H, W, cl) if bcast else skip
        s_ref = residual_sum_numpy(x, full, None if bias is None else
                                   (bias.reshape(1, 1, 1, C) if cl else bias.reshape(1, C, 1, 1)), dt)
        assert np.array_equal(S.view(np.uint8), s_ref.view(np.uint8)), "S differs from numpy's sum"
        ref = _sgn_torch(s_ref, gamma, beta, groups, 1e-5, act, cl, dt)
        assert_within_ulp(Y, ref, 1, f"SGN {np.dtype(dt)}/{np.dtype(pdt)} cl={cl} vs group_norm")


def pin_sgn_invariants(orc):
    rng = np.random.default_rng(32)
    N, C, H, W = 2, 12, 4, 5
    for dt, pdt in [(np.float32, np.float32), (np.float16, np.float16)]:
        x, skip, bias, gamma, beta = _sgn_inputs(rng, dt, pdt, N, C, H, W, 0, True, True)
        kw = dict(groups=3, activation=1, epsilon=1e-5)
        # Broadcast skip == the explicitly expanded skip, bit for bit.
        yb, sb = orc.skip_group_norm(x, gamma, beta, skip, bias, channels_last=0, want_sum=True, **kw)
        yf, sf = orc.skip_group_norm(x, gamma, beta, _expand_skip(skip, N, C, H, W, 0), bias,
                                     channels_last=0, want_sum=True, **kw)
        assert np.array_equal(yb.view(np.uint8), yf.view(np.uint8))
        assert np.array_equal(sb.view(np.uint8), sf.view(np.uint8))
        # (N, 1, 1, C) spelling is the same broadcast.
        y4 = orc.skip_group_norm(x, gamma, beta, skip.reshape(N, 1, 1, C), bias, channels_last=0, **kw)[0]
        assert np.array_equal(y4.view(np.uint8), yb.view(np.uint8))
        # NHWC of the permuted data is the permuted NCHW result.
        xh = np.ascontiguousarray(x.transpose(0, 2, 3, 1))
        yh = orc.skip_group_norm(xh, gamma, beta, skip, bias, channels_last=1, **kw)[0]
        assert_within_ulp(yh, np.ascontiguousarray(yb.transpose(0, 2, 3, 1)), 1, "layout permutation")
        # Requesting S does not change Y.
        y_no = orc.skip_group_norm(x, gamma, beta, skip, bias, channels_last=0, **kw)[0]
        assert np.array_equal(y_no.view(np.uint8), yb.view(np.uint8))
        # Scale invariance (eps = 0, no activation, beta = 0, power of two).
        z = np.zeros_like(beta)
        kw0 = dict(groups=3, activation=0, epsilon=0.0, channels_last=0)
        y1 = orc.skip_group_norm(x, gamma, z, skip, bias, **kw0)[0]
        y2 = orc.skip_group_norm((x * dt(2)).astype(dt), gamma, z, (skip * dt(2)).astype(dt),
                                 (bias * dt(2)).astype(dt), **kw0)[0]
        assert np.array_equal(y1.view(np.uint8), y2.view(np.uint8))
        # groups == C is instance norm; groups == 1 is layer norm over (C, H, W).
        full = _expand_skip(skip, N, C, H, W, 0)
        s = residual_sum_numpy(x, full, bias.reshape(1, C, 1, 1), dt).astype(np.float64)
        st = torch.from_numpy(s)
        g64 = torch.from_numpy(gamma.astype(np.float64))
        b64 = torch.from_numpy(beta.astype(np.float64))
        eps32 = float(np.float32(1e-5))
        yi = orc.skip_group_norm(x, gamma, beta, skip, bias, groups=C, activation=0,
                                 epsilon=1e-5, channels_last=0)[0]
        ref_i = F.instance_norm(st, weight=g64, bias=b64, eps=eps32).numpy().astype(dt)
        assert_within_ulp(yi, ref_i, 1, "groups = C vs instance_norm")
        yl = orc.skip_group_norm(x, gamma, beta, skip, bias, groups=1, activation=0,
                                 epsilon=1e-5, channels_last=0)[0]
        wl = g64.reshape(C, 1, 1).expand(C, H, W)
        bl = b64.reshape(C, 1, 1).expand(C, H, W)
        ref_l = F.layer_norm(st, (C, H, W), wl, bl, eps=eps32).numpy().astype(dt)
        assert_within_ulp(yl, ref_l, 1, "groups = 1 vs layer_norm")
        # gamma = 1, beta = 0, no activation: each group has mean ~0 and
        # variance var/(var + eps) ~ 1 (float32 only: binary16 output is coarse).
        if dt == np.float32:
            ones, zeros = np.ones(C, pdt), np.zeros(C, pdt)
            yn = orc.skip_group_norm(x, ones, zeros, skip, bias, groups=3, activation=0,
                                     epsilon=1e-5, channels_last=0)[0].astype(np.float64)
            per = yn.reshape(N, 3, -1)
            assert np.all(np.abs(per.mean(-1)) < 1e-6)
            sv = s.reshape(N, 3, -1).var(-1)
            assert np.allclose(per.var(-1), sv / (sv + eps32), rtol=1e-6)


# ----------------------------------------------------------------- non-finite values
def _plant_rows(x, k, dt):
    """Row 1 gets +inf, row 2 NaN, row 3 an input pair whose sum overflows dt,
    row 4 both infinities; the other rows stay finite."""
    big = 60000.0 if dt == np.float16 else 3e38
    x[1, 5] = np.inf
    x[2, 7] = np.nan
    x[3, 0] = big
    k[3, 0] = big
    x[4, 1] = np.inf
    x[4, 2] = -np.inf


def pin_non_finite_matches_torch(orc):
    """Infinities and NaNs in the inputs, and sums that overflow the data type.

    The pages say nothing about them, so IEEE arithmetic applied to each
    definition decides the result. The oracle must therefore agree with the
    float64 library routines on the same S:
    - the positions of NaN;
    - the infinities, sign included;
    - every finite output, within one ulp. This covers the zeros that a row
      with an infinite mean square gives its finite elements, and every row or
      group that holds no non-finite value.
    """
    rng = np.random.default_rng(41)
    with np.errstate(all="ignore"):
        for dt, hidden, with_bias in [(np.float32, 40, True), (np.float16, 24, False)]:
            x = rng.standard_normal((6, hidden), dtype=np.float32).astype(dt)
            k = rng.standard_normal((6, hidden), dtype=np.float32).astype(dt)
            g = rng.uniform(0.5, 1.5, hidden).astype(dt)
            be = (0.1 * rng.standard_normal(hidden, dtype=np.float32)).astype(dt)
            b = (0.1 * rng.standard_normal(hidden, dtype=np.float32)).astype(dt) if with_bias else None
            _plant_rows(x, k, dt)
            s_ref = residual_sum_numpy(x, k, b, dt)
            assert np.isinf(s_ref[3, 0]) and np.isnan(s_ref[2, 7]), "planted values not in S"
            st = torch.from_numpy(s_ref.astype(np.float64))
            eps = float(np.float32(1e-6))
            # SSLN: the mean square of rows 1, 3 and 4 is +inf, so their
            # scale is 0: finite elements give (signed) zeros and the
            # infinite ones NaN; row 2 is NaN throughout.
            out, _, inv, s = orc.skip_rms_norm(x, k, g, b, 1e-6, want_inv_std_var=True, want_sum=True)
            assert np.array_equal(np.isnan(s), np.isnan(s_ref)) and \
                np.array_equal(s[~np.isnan(s)].view(np.uint8), s_ref[~np.isnan(s_ref)].view(np.uint8)), \
                "non-finite S differs from numpy's sum"
            y = F.rms_norm(st, (hidden,), torch.from_numpy(g.astype(np.float64)), eps=eps)
            assert_within_ulp(out, y.numpy().astype(dt), 1, f"SSLN {np.dtype(dt)} non-finite output")
            inv_ref = torch.rsqrt(st.pow(2).mean(-1, keepdim=True) + eps)
            assert_within_ulp(inv, inv_ref.numpy().astype(np.float32), 1, "SSLN non-finite inv_std_var")
            # Skip layer norm: the mean of rows 1-4 is non-finite, so their
            # deviations, variance and outputs are NaN.
            out, mean, inv, _ = orc.skip_layer_norm(x, k, g, be, b, 1e-6, want_mean=True,
                                                    want_inv_std_var=True, want_sum=True)
            y = F.layer_norm(st, (hidden,), torch.from_numpy(g.astype(np.float64)),
                             torch.from_numpy(be.astype(np.float64)), eps=eps)
            assert_within_ulp(out, y.numpy().astype(dt), 1, f"SLN {np.dtype(dt)} non-finite output")
            assert_within_ulp(mean, st.mean(-1, keepdim=True).numpy().astype(np.float32), 1,
                              "SLN non-finite mean")
            var = st.var(-1, unbiased=False, keepdim=True)
            assert_within_ulp(inv, torch.rsqrt(var + eps).numpy().astype(np.float32), 1,
                              "SLN non-finite inv_std_var")

        # GatedRMSNorm: X infinite or NaN in some spans; gate +inf (SiLU = inf),
        # -inf (SiLU = -inf * 0 = NaN) and NaN in others.
        for dt in (np.float32, np.float16):
            C = 8
            X = rng.standard_normal((5, 3 * C), dtype=np.float32).astype(dt)
            gate = rng.standard_normal((5, 3 * C), dtype=np.float32).astype(dt)
            scale = rng.uniform(0.5, 1.5, C).astype(dt)
            X[0, 1] = np.inf
            X[1, C + 2] = np.nan
            X[2, 2 * C] = -np.inf
            gate[3, 3] = np.inf
            gate[3, C + 4] = -np.inf
            gate[4, 2 * C + 5] = np.nan
            y = orc.gated_rms_norm(X, scale, gate, 1e-5)
            assert_within_ulp(y, _gated_torch(X, scale, gate, 1e-5, dt), 1, f"gated {np.dtype(dt)} non-finite")

        # SkipGroupNorm: a group's non-finite mean or variance makes the whole
        # group NaN (SiLU keeps NaN); the other groups of the image and the
        # other images are untouched.
        for dt, pdt, cl, bcast, act in [(np.float16, np.float32, 1, False, 1),
                                        (np.float32, np.float16, 0, True, 0),
                                        (np.float32, np.float32, 1, False, 1)]:
            N, C, H, W, groups = 3, 12, 3, 4, 3
            x, skip, bias, gamma, beta = _sgn_inputs(rng, dt, pdt, N, C, H, W, cl, bcast, True)
            big = 60000.0 if dt == np.float16 else 3e38
            at = (lambda n, c, h, w: (n, h, w, c)) if cl else (lambda n, c, h, w: (n, c, h, w))
            x[at(0, 5, 1, 2)] = np.inf                 # image 0, group 1
            x[at(1, 0, 2, 3)] = np.nan                 # image 1, group 0
            x[at(1, 11, 0, 0)] = big                   # image 1, group 2: S overflows
            if bcast:
                skip[1, 11] = big
            else:
                skip[at(1, 11, 0, 0)] = big
            x[at(2, 4, 0, 1)] = np.inf                 # image 2, group 1: both infinities
            x[at(2, 6, 2, 0)] = -np.inf
            Y, S = orc.skip_group_norm(x, gamma, beta, skip, bias, groups=groups, activation=act,
                                       epsilon=1e-5, channels_last=cl, want_sum=True)
            full = _expand_skip(skip, N, C, H, W, cl) if bcast else skip
            s_ref = residual_sum_numpy(x, full, bias.reshape(1, 1, 1, C) if cl else bias.reshape(1, C, 1, 1), dt)
            assert np.array_equal(np.isnan(S), np.isnan(s_ref)) and \
                np.array_equal(S[~np.isnan(S)].view(np.uint8), s_ref[~np.isnan(s_ref)].view(np.uint8)), \
                "non-finite S differs from numpy's sum"
            ref = _sgn_torch(s_ref, gamma, beta, groups, 1e-5, act, cl, dt)
            assert_within_ulp(Y, ref, 1, f"SGN {np.dtype(dt)} cl={cl} non-finite vs group_norm")
            ys = Y.reshape(N, H * W, C) if cl else np.moveaxis(Y.reshape(N, C, H * W), 1, 2)
            ys = ys.reshape(N, H * W, groups, C // groups)
            nan_groups = [(0, 1), (1, 0), (1, 2), (2, 1)]
            for n in range(N):
                for gi in range(groups):
                    blk = ys[n, :, gi]
                    assert np.isnan(blk).all() == ((n, gi) in nan_groups), f"group ({n}, {gi})"
                    assert np.isfinite(blk).all() == ((n, gi) not in nan_groups), f"group ({n}, {gi})"


PINS = [pin_hand_cases, pin_f16_decode_exhaustive, pin_f32_to_f16_structured,
        pin_f64_to_f16_ties, pin_ssln_matches_torch, pin_ssln_invariants,
        pin_sln_matches_torch, pin_sln_invariants,
        pin_gated_matches_torch, pin_gated_invariants, pin_sgn_matches_torch,
        pin_sgn_invariants, pin_non_finite_matches_torch]
