"""The oracle's pins have teeth: each planted mistake fails at least one.

Every mutant is a one-line edit of a copy of oracle.c (a dropped term, a
wrong sign, divisor, index or constant), compiled with gcc into a temporary
directory and run through the pin tests.  The edits live only here and only
on the CPU; oracle.c itself is never changed.
"""
import inspect

import pytest

import oracle as O
from tests import test_oracle_pins as pins
from tests import test_oracle_allreduce_pins as allreduce_pins
from tests import test_oracle_gemm_pins as gemm_pins
from tests import test_oracle_swiglu_pins as swiglu_pins

MUTANTS = {
    "dropped_eps": ("sqrt(ms + (double)eps)", "sqrt(ms)"),
    "divisor_h_minus_1": ("sum / (double)n", "sum / (double)(n - 1)"),
    "variance_over_all_channels": ("ms = mean_square(variance_size, r);",
                                   "ms = mean_square(hidden, r);"),
    "variance_divisor_hidden": ("ms = mean_square(variance_size, r);",
                                "ms = mean_square(variance_size, r) * variance_size / hidden;"),
    "abs_instead_of_r": ("y[j] = r[j] * inv * w;", "y[j] = fabs(r[j]) * inv * w;"),
    "weight_index_shift": ("orc_decode16(dtype, weight[j])",
                           "orc_decode16(dtype, weight[(j + 1) % hidden])"),
    "unrounded_residual": ("r[j] = orc_decode16(dtype, r16[j]);", "r[j] = sum;"),
    "residual_added_twice_x": ("orc_decode16(dtype, res[j])", "orc_decode16(dtype, x[j])"),
    "ties_away_from_zero": ("frac == 0.5 && fmod(lo, 2.0) != 0.0", "frac == 0.5"),
    "no_fp8_saturation": ("if (a >= 448.0) {", "if (a >= 480.0) {"),
    "fp8_subnormal_edge": ("if (e < -6) {", "if (e < -7) {"),
    "fnuz_dynamic_max": ("scale = (float)(amax / 448.0);", "scale = (float)(amax / 240.0);"),
    "static_scale_multiplied": ("orc_e4m3_encode(y[j] / (double)s)",
                                "orc_e4m3_encode(y[j] * (double)s)"),
    "static_quotient_rounded_to_fp32": ("orc_e4m3_encode(y[j] / (double)s)",
                                        "orc_e4m3_encode((double)(float)(y[j] / (double)s))"),
    "dynamic_quotient_rounded_to_fp32": ("orc_e4m3_encode(y[j] / (double)scale)",
                                         "orc_e4m3_encode((double)(float)(y[j] / (double)scale))"),
    "row_stride_ignored": ("const uint16_t *xi = x + i * x_stride;",
                           "const uint16_t *xi = x + i * hidden;"),
    "fp16_bias": ("f.bias = 15;", "f.bias = 16;"),
    "subnormal_scale": ("ldexp((double)m, 1 - f.bias - f.man_bits)",
                        "ldexp((double)m, -f.bias - f.man_bits)"),
    "square_not_squared": ("sum += r[j] * r[j];", "sum += fabs(r[j]);"),
    "e4m3_bias": ("ldexp((double)(8 + m), e - 7 - 3)", "ldexp((double)(8 + m), e - 8 - 3)"),
    "overflow_not_inf": ("if (e + f.bias >= emax_field) {", "if (e + f.bias > emax_field) {"),
    "silu_sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "silu_no_sigmoid": ("return g / (1.0 + exp(-g));", "return g;"),
    "silu_negative_sign": ("const double e = exp(g);", "const double e = exp(-g);"),
    "silu_negative_no_denominator": ("return g * e / (1.0 + e);", "return g * e;"),
    "gate_up_swapped": ("y[j] = orc_silu(g) * u;", "y[j] = orc_silu(u) * g;"),
    "up_row_stride": ("up[i * up_stride + j]", "up[i * gate_stride + j + 0 * up_stride]"),
    "sum_in_double": ("float total = (float)orc_decode16(dtype, parts[0][i * parts_stride + j]);",
                      "double total = (float)orc_decode16(dtype, parts[0][i * parts_stride + j]);"),
    "sum_drops_last_part": ("for (g = 1; g < nparts; g++) {\n                total",
                            "for (g = 1; g < nparts - 1; g++) {\n                total"),
    "sum_wrong_stride": ("total = total + (float)orc_decode16(dtype, parts[g][i * parts_stride + j]);",
                         "total = total + (float)orc_decode16(dtype, parts[g][i * hidden + j]);"),
    "gemm_b_transposed": ("orc_e4m3_decode(b[j * ldb + t])", "orc_e4m3_decode(b[t * ldb + j])"),
    "gemm_scale_b_per_row_ignored": ("double scale_b = (double)(b_per_row ? sb[j] : sb[0]);",
                                     "double scale_b = (double)sb[0];"),
    "gemm_k_off_by_one": ("for (t = 0; t < k; t++) {\n                double p",
                          "for (t = 1; t < k; t++) {\n                double p"),
    "gemm_a_row_stride": ("orc_e4m3_decode(a[i * lda + t])", "orc_e4m3_decode(a[i * k + t])"),
    "glu_dynamic_scale_of_u": ("double u = orc_decode16(dtype, up[i * up_stride + j]);",
                               "double u = orc_decode16(dtype, up[i * up_stride + j]) * 2.0;"),
}


def _pin_functions():
    fns = []
    members = inspect.getmembers(pins, inspect.isfunction) + \
        inspect.getmembers(swiglu_pins, inspect.isfunction) + \
        inspect.getmembers(gemm_pins, inspect.isfunction) + \
        inspect.getmembers(allreduce_pins, inspect.isfunction)
    for name, fn in members:
        if not name.startswith("test_"):
            continue
        if "exhaustive" in name:
            continue  # minute-long brute force: run once by its own module
        params = inspect.signature(fn).parameters
        marks = getattr(fn, "pytestmark", [])
        calls = [()]
        for m in marks:
            if m.name == "parametrize":
                argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else m.args[0]
                new = []
                for c in calls:
                    for v in m.args[1]:
                        vals = v if len(argnames) > 1 else (v,)
                        new.append(c + tuple(zip(argnames, vals)))
                calls = new
        for c in calls:
            kwargs = dict(c)
            if set(params) - {"orc"} - set(kwargs):
                continue
            fns.append((name, fn, kwargs))
    # cheap pins first so most mutants stop early
    slow = ("residual_sum", "round_trips", "midpoints", "random")
    fns.sort(key=lambda t: any(s in t[0] for s in slow))
    return fns


def _compile_mutant(tmp_path, name, old, new):
    src = open(O._SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor must occur exactly once"
    mdir = tmp_path / name
    mdir.mkdir()
    csrc = mdir / "oracle.c"
    csrc.write_text(src.replace(old, new))
    (mdir / "oracle.h").write_text(open(O._HDR).read())
    return O.bind(O.build(str(csrc), str(mdir / "liboracle.so")))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    orc = O.Oracle(_compile_mutant(tmp_path, name, old, new))
    caught = []
    for fname, fn, kwargs in _pin_functions():
        try:
            fn(orc=orc, **kwargs)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(fname)
            break
    assert caught, f"no pin catches mutant {name}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    orc = O.Oracle(_compile_mutant(tmp_path, "none", "#include <stdlib.h>", "#include <stdlib.h>"))
    for fname, fn, kwargs in _pin_functions():
        fn(orc=orc, **kwargs)
