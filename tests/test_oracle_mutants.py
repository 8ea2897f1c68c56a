"""The oracle pins must catch plausible mistakes.

Each case plants one slip in a private copy of the oracle's C source, builds it
with gcc into a temporary library, points the oracle module at it and runs the
pin tests: at least one pin has to fail.  Everything here runs on the CPU; the
real oracle library is restored afterwards.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as oracle_build
from tests import test_oracle_pins as pins
from tests import test_oracle_quant_pins as qpins
from tests import test_oracle_bwd_pins as bpins
from tests import test_oracle_ln_pins as lpins
from tests import test_oracle_kv_pins as kpins
from tests import test_oracle_unrounded_pins as upins

MUTANTS = [
    ("eps dropped", "sqrt(mean + (double)eps)", "sqrt(mean)"),
    ("eps outside the root", "r = 1.0 / sqrt(mean + (double)eps);", "r = 1.0 / sqrt(mean) + (double)eps;"),
    ("divisor hidden - 1", "mean = s / (double)hidden;", "mean = s / (double)(hidden > 1 ? hidden - 1 : 1);"),
    ("no square root", "r = 1.0 / sqrt(mean + (double)eps);", "r = 1.0 / (mean + (double)eps);"),
    ("sum of |x| instead of x^2", "s += v[j] * v[j];", "s += fabs(v[j]);"),
    ("weight dropped", "v[j] * r * load_elem(w, j, dtype)", "v[j] * r"),
    ("weight index shifted", "v[j] * r * load_elem(w, j, dtype)", "v[j] * r * load_elem(w, (j + 1) % hidden, dtype)"),
    ("sign lost", "v[j] * r * load_elem(w, j, dtype)", "fabs(v[j]) * r * load_elem(w, j, dtype)"),
    ("rows and columns transposed", "load_elem(x, i * hidden + j, dtype)", "load_elem(x, j * rows + i, dtype)"),
    ("truncating rounding", "nearbyint(a / spacing)", "floor(a / spacing)"),
    ("ties away from zero", "nearbyint(a / spacing)", "round(a / spacing)"),
    ("bf16 rounded via float32", "a = fabs(v);", "a = fabs((double)(float)v);"),
    ("subnormal spacing wrong", "if (e2 < -126) e2 = -126;", ""),
    ("residual subtracted", "load_elem(x, k, dtype) + load_elem(residual, k, dtype)",
     "load_elem(x, k, dtype) - load_elem(residual, k, dtype)"),
    ("unrounded residual sum normalised", "v[j] = load_elem(h_out, k, dtype);", "v[j] = sum;"),
    ("rounded before the weight multiply",
     "store_elem(out, out_off + j, v[j] * r * load_elem(w, j, dtype), out_dtype);",
     "store_elem(out, out_off + j, (dtype == ORACLE_BF16 ? "
     "(double)oracle_bf16_back(oracle_round_bf16(v[j] * r)) : (double)(float)(v[j] * r)) "
     "* load_elem(w, j, dtype), out_dtype);"),
]

MUTANTS += [
    ("int8 full scale 128", "qtype == ORACLE_QUANT_INT8 ? 127.0 : 448.0", "qtype == ORACLE_QUANT_INT8 ? 128.0 : 448.0"),
    ("fp8 full scale 240", "qtype == ORACLE_QUANT_INT8 ? 127.0 : 448.0", "qtype == ORACLE_QUANT_INT8 ? 127.0 : 240.0"),
    ("truncating quantisation", "double c = nearbyint(t);", "double c = trunc(t);"),
    ("codes from the unscaled output", "double t = amax > 0.0 ? y[j] / scale : 0.0;",
     "double t = amax > 0.0 ? y[j] * 100.0 : 0.0;"),
    ("scale not divided by the full scale", "scale = amax / qmax;\n        scale_out[i] = (float)scale;",
     "scale = amax / qmax;\n        scale_out[i] = (float)amax;"),
    ("quantising the bf16-rounded output", "y[j] = v[j] * r * load_elem(w, j, dtype);",
     "y[j] = (double)oracle_bf16_back(oracle_round_bf16(v[j] * r * load_elem(w, j, dtype)));"),
    ("residual ignored by the quantiser", "            if (residual) {\n                store_elem(h_out, k, load_elem(x, k, dtype) + load_elem(residual, k, dtype), dtype);",
     "            if (residual) {\n                store_elem(h_out, k, load_elem(x, k, dtype), dtype);"),
    ("fp8 exponent bias 8", "code = ((e2 + 7) << 3)", "code = ((e2 + 8) << 3)"),
    ("fp8 subnormal spacing wrong", "if (e2 < -6) e2 = -6;", "if (e2 < -7) e2 = -7;"),
    ("fp8 ties away from zero", "m = nearbyint(a / spacing) * spacing;\n    if (m > 448.0) m = 448.0;",
     "m = round(a / spacing) * spacing;\n    if (m > 448.0) m = 448.0;"),
]

MUTANTS += [
    ("bwd r squared in the radial term", "v * r * r * r * c / (double)hidden", "v * r * r * c / (double)hidden"),
    ("bwd radial term without 1/H", "v * r * r * r * c / (double)hidden", "v * r * r * r * c"),
    ("bwd radial term added", "r * g * load_elem(w, j, dtype) - v * r", "r * g * load_elem(w, j, dtype) + v * r"),
    ("bwd weight missing from c", "c += load_elem(dy, i * hidden + j, dtype) * load_elem(w, j, dtype) * v;",
     "c += load_elem(dy, i * hidden + j, dtype) * v;"),
    ("bwd weight missing from the direct term", "store_elem(dx, i * hidden + j, r * g * load_elem(w, j, dtype)",
     "store_elem(dx, i * hidden + j, r * g"),
    ("bwd eps dropped", "r = 1.0 / sqrt(s / (double)hidden + (double)eps);", "r = 1.0 / sqrt(s / (double)hidden);"),
    ("bwd dw without r", "acc[j] += g * v * r;", "acc[j] += g * v;"),
    ("bwd dw times the weight", "acc[j] += g * v * r;", "acc[j] += g * v * r * load_elem(w, j, dtype);"),
    ("bwd dw keeps only the last row", "acc[j] += g * v * r;", "acc[j] = g * v * r;"),
    ("bwd dy read transposed", "double g = load_elem(dy, i * hidden + j, dtype);",
     "double g = load_elem(dy, j * rows + i, dtype);"),
]

MUTANTS += [
    ("ln variance divisor H - 1", "inv = 1.0 / sqrt(q / (double)hidden + (double)eps);",
     "inv = 1.0 / sqrt(q / (double)(hidden > 1 ? hidden - 1 : 1) + (double)eps);"),
    ("ln eps outside the root", "inv = 1.0 / sqrt(q / (double)hidden + (double)eps);",
     "inv = 1.0 / sqrt(q / (double)hidden) + (double)eps;"),
    ("ln mean not subtracted", "double v = load_elem(gamma, j, dtype) * (load_elem(x, i * hidden + j, dtype) - mu) * inv;",
     "double v = load_elem(gamma, j, dtype) * load_elem(x, i * hidden + j, dtype) * inv;"),
    ("ln beta dropped", "if (beta) v += load_elem(beta, j, dtype);", "if (beta) v += 0.0;"),
    ("ln gamma added as the bias", "if (beta) v += load_elem(beta, j, dtype);", "if (beta) v += load_elem(gamma, j, dtype);"),
    ("ln uncentred fp32 variance",
     "            double d = load_elem(x, i * hidden + j, dtype) - mu;\n            q += d * d;\n        }\n"
     "        inv = 1.0 / sqrt(q / (double)hidden + (double)eps);",
     "            float d = (float)load_elem(x, i * hidden + j, dtype);\n            q += (double)(d * d);\n        }\n"
     "        inv = 1.0 / sqrt((double)((float)(q / (double)hidden) - (float)(mu * mu)) + (double)eps);"),
    ("ln mean read transposed", "for (j = 0; j < hidden; ++j) s += load_elem(x, i * hidden + j, dtype);",
     "for (j = 0; j < hidden; ++j) s += load_elem(x, j * rows + i, dtype);"),
]

MUTANTS += [
    ("kv rotation sign", "store_elem(rope_cache, out + ia, a * c - b * sn, out_dtype);",
     "store_elem(rope_cache, out + ia, a * c + b * sn, out_dtype);"),
    ("kv cos and sin swapped", "const double c = (double)cos_t[pos * half + j], sn = (double)sin_t[pos * half + j];",
     "const double c = (double)sin_t[pos * half + j], sn = (double)cos_t[pos * half + j];"),
    ("kv halves paired as adjacent elements",
     "const int64_t ia = rope_style ? 2 * j : j, ib = rope_style ? 2 * j + 1 : j + half;",
     "const int64_t ia = 2 * j, ib = 2 * j + 1;"),
    ("kv table row off by one", "const double c = (double)cos_t[pos * half + j], sn = (double)sin_t[pos * half + j];",
     "const int64_t p1 = pos + 1 < max_pos ? pos + 1 : pos;\n"
     "                const double c = (double)cos_t[p1 * half + j], sn = (double)sin_t[p1 * half + j];"),
    ("kv slot ignored", "store_elem(norm_cache, (slot * heads + h) * norm_dim + j,",
     "store_elem(norm_cache, (t * heads + h) * norm_dim + j,"),
    ("kv eps dropped", "r = 1.0 / sqrt(s / (double)norm_dim + (double)eps);", "r = 1.0 / sqrt(s / (double)norm_dim);"),
    ("kv gamma dropped", "load_elem(kv, in + j, dtype) * r * load_elem(gamma, j, dtype), out_dtype);",
     "load_elem(kv, in + j, dtype) * r, out_dtype);"),
    ("kv every head read from head 0", "const int64_t in = (t * heads + h) * d;", "const int64_t in = t * heads * d;"),
]

MUTANTS += [
    ("unrounded output passed through float32", "memcpy((char *)base + 8 * i, &v, 8);",
     "v = (double)(float)v;\n        memcpy((char *)base + 8 * i, &v, 8);"),
    ("array bf16 rounding via float32", "for (i = 0; i < n; ++i) out[i] = oracle_round_bf16(v[i]);",
     "for (i = 0; i < n; ++i) out[i] = oracle_round_bf16((double)(float)v[i]);"),
    ("unrounded output without the weight", "store_elem(out, out_off + j, v[j] * r * load_elem(w, j, dtype), out_dtype);",
     "store_elem(out, out_off + j, out_dtype == ORACLE_F64 ? v[j] * r : v[j] * r * load_elem(w, j, dtype), out_dtype);"),
    ("unrounded dx without the radial term",
     "r * g * load_elem(w, j, dtype) - v * r * r * r * c / (double)hidden,\n                           out_dtype);",
     "r * g * load_elem(w, j, dtype) - (out_dtype == ORACLE_F64 ? 0.0 : v * r * r * r * c / (double)hidden),\n"
     "                           out_dtype);"),
    ("unrounded layernorm without beta", "if (beta) v += load_elem(beta, j, dtype);",
     "if (beta && out_dtype != ORACLE_F64) v += load_elem(beta, j, dtype);"),
    ("unrounded rope sign", "store_elem(rope_cache, out + ib, a * sn + b * c, out_dtype);",
     "store_elem(rope_cache, out + ib, out_dtype == ORACLE_F64 ? b * c - a * sn : a * sn + b * c, out_dtype);"),
]

HELPER = """
static float oracle_bf16_back(uint16_t b) { uint32_t u = (uint32_t)b << 16; float f; memcpy(&f, &u, 4); return f; }
"""

PIN_TESTS = [
    (pins.test_round_bf16_matches_exact_rational_rounding, {}),
    (pins.test_round_bf16_ties_go_to_even, {}),
    (pins.test_hand_computed_four_element_example, {}),
    (pins.test_exact_example_every_dtype_bitwise, {}),
    (pins.test_constant_row_closed_form, dict(c=1e-3, eps=pins.EPS6, dtype="f32")),
    (pins.test_constant_row_closed_form, dict(c=3.0, eps=pins.EPS5, dtype="bf16")),
    (pins.test_single_column_rows, {}),
    (pins.test_power_of_two_scale_invariance_bitwise, dict(k=3)),
    (pins.test_row_independence_and_layout, {}),
    (pins.test_zero_row_and_signs, {}),
    (pins.test_rms_identity, {}),
    (pins.test_brute_force_tiny_rows, dict(dtype="bf16")),
    (pins.test_brute_force_tiny_rows, dict(dtype="f32")),
    (pins.test_residual_sum_rounded_once, dict(dtype="bf16")),
    (pins.test_residual_normalises_the_rounded_sum, {}),
    (pins.test_residual_special_cases_reduce_to_plain, {}),
    (qpins.test_e4m3_rounding_matches_exact_rational, {}),
    (qpins.test_e4m3_ties_go_to_even, {}),
    (qpins.test_hand_worked_codes, dict(qtype=0)),
    (qpins.test_hand_worked_codes, dict(qtype=1)),
    (qpins.test_codes_are_the_exact_rational_closed_form, dict(qtype=0, dtype="bf16")),
    (qpins.test_codes_are_the_exact_rational_closed_form, dict(qtype=1, dtype="bf16")),
    (qpins.test_scale_closed_form_constant_row, dict(qtype=0)),
    (qpins.test_row_max_maps_to_full_scale_and_zero_row, dict(qtype=1)),
    (qpins.test_fused_quant_uses_the_rounded_sum, dict(qtype=0)),
    (bpins.test_matches_decimal_central_differences, dict(dtype="f32", hidden=5)),
    (bpins.test_matches_decimal_central_differences, dict(dtype="bf16", hidden=8)),
    (bpins.test_single_column_closed_form, dict(dtype="f32")),
    (bpins.test_orthogonal_to_x_without_eps, {}),
    (bpins.test_eps_component_along_x, {}),
    (bpins.test_power_of_two_scaling_without_eps, dict(k=5)),
    (bpins.test_weight_gradient_identity, {}),
    (bpins.test_linear_in_dy_and_zero_gradient, {}),
    (bpins.test_rows_independent_and_dw_sums_rows, {}),
    (lpins.test_matches_torch_layer_norm_in_float64, dict(dtype="f32", with_beta=True)),
    (lpins.test_two_columns_closed_form, dict(dtype="f32")),
    (lpins.test_constant_rows_and_single_column_give_beta, dict(dtype="bf16")),
    (lpins.test_shift_invariance_bitwise, {}),
    (lpins.test_scale_and_sign_invariance_bitwise, {}),
    (lpins.test_standardised_moments, {}),
    (lpins.test_rows_independent_and_layout, {}),
    (lpins.test_pages_layernorm_test_case, {}),
    (kpins.test_norm_part_is_the_rmsnorm_oracle, dict(dtype="f32", style=1)),
    (kpins.test_rope_part_is_a_complex_multiplication, dict(dtype="f32", style=0)),
    (kpins.test_rope_part_is_a_complex_multiplication, dict(dtype="bf16", style=1)),
    (kpins.test_position_zero_is_the_identity, dict(style=1)),
    (kpins.test_quarter_turn_moves_exactly_one_pair, dict(style=0)),
    (kpins.test_quarter_turn_moves_exactly_one_pair, dict(style=1)),
    (kpins.test_rotation_preserves_pair_lengths, {}),
    (kpins.test_scatter_rows_and_skips, dict(dtype="bf16")),
    (upins.test_round_arrays_match_exact_rational_rounding, {}),
    (upins.test_unrounded_hand_example, dict(dtype="f32")),
    (upins.test_unrounded_brute_force_tiny_rows, dict(dtype="bf16")),
    (upins.test_rounding_the_unrounded_output_gives_the_rounded_output, dict(dtype="bf16")),
    (upins.test_unrounded_backward_matches_decimal_central_differences, {}),
    (upins.test_unrounded_layernorm_two_columns, {}),
    (upins.test_unrounded_kv_parts, dict(style=oracle.ROPE_PAIRS)),
]


def _build_mutant(src: str, tmpdir: str) -> str:
    path = os.path.join(tmpdir, "mutant.c")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmpdir, "libmutant.so")
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", lib, path, "-lm"], check=True, capture_output=True)
    return lib


def _load_mutant(lib_path):
    import ctypes
    saved = oracle._lib
    oracle._lib = None
    real = oracle_build.LIB
    oracle_build.LIB = lib_path
    try:
        lib = oracle._load()
    finally:
        oracle_build.LIB = real
        oracle._lib = saved
    assert isinstance(lib, ctypes.CDLL)
    return lib


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    with open(oracle_build.SRC) as f:
        src = f.read()
    assert old in src, "mutation anchor not found: %r" % old
    mutated = src.replace(old, new, 1)
    mutated = mutated.replace("#define ORACLE_BF16 1", "#define ORACLE_BF16 1\n" + HELPER, 1)
    with tempfile.TemporaryDirectory() as d:
        lib = _load_mutant(_build_mutant(mutated, d))
        saved = oracle._lib
        oracle._lib = lib
        failed = []
        try:
            for fn, kw in PIN_TESTS:
                try:
                    fn(**kw)
                except (AssertionError, RuntimeError, ValueError, OverflowError, ZeroDivisionError):
                    failed.append(fn.__name__)
        finally:
            oracle._lib = saved
    assert failed, "no pin caught the mutant %r" % name


def test_unmodified_copy_passes_every_pin():
    """Control for the harness: a rebuilt, unmodified copy fails no pin."""
    with open(oracle_build.SRC) as f:
        src = f.read()
    with tempfile.TemporaryDirectory() as d:
        lib = _load_mutant(_build_mutant(src, d))
        saved = oracle._lib
        oracle._lib = lib
        try:
            for fn, kw in PIN_TESTS:
                fn(**kw)
        finally:
            oracle._lib = saved
