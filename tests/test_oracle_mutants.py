"""Planted mistakes: every altered build of the oracle must fail a pin.

Each mutation is a plausible slip (a dropped term, a wrong sign, a wrong
index or divisor, swapped operands, a rounding tie broken the wrong way).  It
is applied to a copy of the C source, compiled with gcc on the CPU into a
temporary library, and the pins of ``pins.py`` are run against that build.
A mutation that no pin catches means the pins leave that part of the oracle
unchecked, and the test fails.  All mutations keep every array access in
bounds.  (Slips that leave the computed function unchanged, such as a
consistent transpose of the two spatial axes, are not listed: no test can
or should catch them.)
"""

import pytest

import oracle
from pins import PINS

MUTATIONS = [
    ("rms divisor hidden-1", "sum_sq / (double)hidden", "sum_sq / (double)(hidden - 1)"),
    ("bias subtracted", "if (has_bias) s = s + bias;", "if (has_bias) s = s - bias;"),
    ("bias dropped", "if (has_bias) s = s + bias;", "if (has_bias) s = s;"),
    ("sum not rounded to T", "return round_f32_to_type(T, s);", "return s;"),
    ("gamma reversed", "(double)load_f32(T, gamma, j));",
     "(double)load_f32(T, gamma, hidden - 1 - j));"),
    ("ssln epsilon dropped", "1.0 / sqrt(mean_sq + eps)", "1.0 / sqrt(mean_sq)"),
    ("inv_std_var is RMS", "inv_std_var[r] = (float)inv_rms;",
     "inv_std_var[r] = (float)(1.0 / inv_rms);"),
    ("ln variance unbiased", "ssd / (double)hidden + eps", "ssd / (double)(hidden - 1) + eps"),
    ("ln mean not removed", "double y = (s[j] - mu) * inv", "double y = s[j] * inv"),
    ("ln beta scaled by gamma", "if (beta) y += (double)load_f32(T, beta, j);",
     "if (beta) y += (double)load_f32(T, beta, j) * (double)load_f32(T, gamma, j);"),
    ("ln mean output zero", "if (mean) mean[r] = (float)mu;", "if (mean) mean[r] = 0.0f;"),
    ("ln epsilon dropped", "sqrt(ssd / (double)hidden + eps)", "sqrt(ssd / (double)hidden)"),
    ("gated epsilon dropped", "sqrt(sum_sq / (double)C + eps)", "sqrt(sum_sq / (double)C)"),
    ("gated scale index fixed", "(double)load_f32(T, scale, j)", "(double)load_f32(T, scale, 0)"),
    ("silu sign", "return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    ("gate and x swapped", "store_f64(T, Y, base + j, x * inv_rms * sc * silu(g));",
     "store_f64(T, Y, base + j, g * inv_rms * sc * silu(x));"),
    ("group variance unbiased", "const double var = sq / count;",
     "const double var = sq / (count - 1.0);"),
    ("gamma and beta swapped", "const double gm = (double)load_f32(M, gamma, c);",
     "const double gm = (double)load_f32(M, beta, c);"),
    ("group eps dropped", "1.0 / sqrt(var + eps)", "1.0 / sqrt(var)"),
    ("broadcast ignores batch", "skip_broadcast ? n * C + c : i", "skip_broadcast ? c : i"),
    ("nhwc read as nchw", "return ((n * H + h) * W + w) * C + c;",
     "return ((n * C + c) * H + h) * W + w;"),
    ("activation before affine", "double y = gm * (s[i] - mean) * rstd + bt;\n"
     "                        if (activation == 1) y = silu(y);",
     "double y = (s[i] - mean) * rstd;\n"
     "                        if (activation == 1) y = silu(y);\n"
     "                        y = gm * y + bt;"),
    ("group mean off by one", "const double mean = sum / count;",
     "const double mean = sum / (count + 1.0);"),
    ("gated squares dropped", "sum_sq += x * x;", "sum_sq += x;"),
    ("gated rms from the gate", "double x = (double)load_f32(T, X, base + j);\n            sum_sq",
     "double x = (double)load_f32(T, gate, base + j);\n            sum_sq"),
    ("group bias fixed channel", "bias ? load_f32(T, bias, c) : 0.0f", "bias ? load_f32(T, bias, 0) : 0.0f"),
    ("group activation ignored", "if (activation == 1) y = silu(y);\n                        store_f64",
     "if (activation == 2) y = silu(y);\n                        store_f64"),
    ("group mean over one channel",
     "for (int64_t c = g * cpg; c < (g + 1) * cpg; ++c)\n                for (int64_t h = 0; h < H; ++h)\n"
     "                    for (int64_t w = 0; w < W; ++w)\n                        sum +=",
     "for (int64_t c = g * cpg; c < g * cpg + 1; ++c)\n                for (int64_t h = 0; h < H; ++h)\n"
     "                    for (int64_t w = 0; w < W; ++w)\n                        sum +="),
    ("gamma by group", "const double gm = (double)load_f32(M, gamma, c);",
     "const double gm = (double)load_f32(M, gamma, g);"),
    ("skip added twice", "float sv = residual_sum(T, load_f32(T, X, i), load_f32(T, skip, k),",
     "float sv = residual_sum(T, load_f32(T, X, i) + load_f32(T, skip, k), load_f32(T, skip, k),"),
    ("rounding ties away", "if (frac < 0.5) return fl;\n    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;",
     "if (frac < 0.5) return fl;\n    return fl + 1.0;"),
    ("overflow threshold", "if (a >= 65520.0)", "if (a >= 131072.0)"),
    ("subnormal quantum", "round_half_even(a * ldexp(1.0, 24))", "round_half_even(a * ldexp(1.0, 23))"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / f"libmutant_{abs(hash(name))}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
