"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/qkv_oracle.c (on the CPU, in a
temporary directory), builds it with the oracle's flags, routes the oracle's
Python front end to that build and runs the pins of test_oracle_pins.py.  At
least one pin must fail for every planted mistake; the pins that caught it are
listed in the assertion message of a survivor.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_norm_pins as npins
import test_oracle_pins as pins
import test_oracle_fp8_pins as fpins
import test_oracle_proj_pins as ppins
import test_oracle_rope_variants as rpins
from qkv_bias_rope_amd import workloads as wl

SRC = os.path.join(os.path.dirname(oracle.__file__), "qkv_oracle.c")

# (name, [(old, new), ...]): every occurrence of `old` is replaced (the same
# mistake in both chains where they share a line); each `old` must occur.
MUTATIONS = [
    ("drop q bias", [("\n    oracle_add_bias(q, bq, nt, nqt, ld_q);\n", "\n"),
                     ("        oracle_add_bias(q, bq, nt, nqt, ld_q);\n", "        ;\n")]),
    ("drop v bias", [("\n    oracle_add_bias(v, bv, nt, nkt, ld_v);\n", "\n"),
                     ("        oracle_add_bias(v, bv, nt, nkt, ld_v);\n", "        ;\n")]),
    ("bias subtracted", [("x[t * ld + j] = x[t * ld + j] + b[j];", "x[t * ld + j] = x[t * ld + j] - b[j];")]),
    ("rotation sign flipped", [("(float)((double)x0 * c - (double)x1 * s)", "(float)((double)x0 * c + (double)x1 * s)")]),
    ("reverse rotation", [("(float)((double)x0 * c - (double)x1 * s)", "(float)((double)x0 * c + (double)x1 * s)"),
                          ("(float)((double)x0 * s + (double)x1 * c)", "(float)(-(double)x0 * s + (double)x1 * c)")]),
    ("cos and sin swapped", [("float c = (float)cos((double)a);", "float c = (float)sin((double)a);"),
                             ("float s = (float)sin((double)a);", "float s = (float)cos((double)a);")]),
    ("interleaved pairing", [("float x0 = row[i];", "float x0 = row[2 * i];"),
                             ("float x1 = row[i + half];", "float x1 = row[2 * i + 1];"),
                             ("row[i]        = (float)", "row[2 * i]    = (float)"),
                             ("row[i + half] = (float)", "row[2 * i + 1] = (float)")]),
    ("exponent 1i/hd", [("-(2.0 * (double)i) / (double)head_dim", "-(1.0 * (double)i) / (double)head_dim")]),
    ("inverse frequency not inverted", [("-(2.0 * (double)i) / (double)head_dim", "(2.0 * (double)i) / (double)head_dim")]),
    ("first token's position for all", [("float a = (float)pos[t] * inv[i];", "float a = (float)pos[0] * inv[i];")]),
    ("position off by one", [("float a = (float)pos[t] * inv[i];", "float a = (float)(pos[t] + 1) * inv[i];")]),
    ("k not rotated", [("    oracle_rope_neox(k, nt, ld_k, n_kv_head, head_dim, pos, inv);\n", "")]),
    ("v rotated too", [("    oracle_rope_neox(k, nt, ld_k, n_kv_head, head_dim, pos, inv);\n",
                        "    oracle_rope_neox(k, nt, ld_k, n_kv_head, head_dim, pos, inv);\n"
                        "    oracle_rope_neox(v, nt, ld_v, n_kv_head, head_dim, pos, inv);\n")]),
    ("V row from k", [("    oracle_store_rows(v, nt, ld_v, nkt, pos, slot, n_ctx, n_slots,",
                       "    oracle_store_rows(k, nt, ld_k, nkt, pos, slot, n_ctx, n_slots,")]),
    ("f16 truncates", [("    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u)))", "    if (0)")]),
    ("f16 ties away from zero", [("(rem == 0x1000u && (h & 1u))", "(rem == 0x1000u)")]),
    ("f16 subnormals flushed", [("if (exp < 102)", "if (exp < 113)")]),
    ("f16 overflow saturates", [("        return (uint16_t)(sign | 0x7c00u);\n\n    if (e16 <= 0)",
                                 "        return (uint16_t)(sign | 0x7bffu);\n\n    if (e16 <= 0)")]),
    ("slot ignored", [("return s * n_ctx + p;", "return p;")]),
    ("position bound off by one", [("if (p < 0 || p >= n_ctx)", "if (p < 0 || p > n_ctx)")]),
    ("slot bound missing", [("if (s < 0 || s >= n_slots)", "if (s < 0)")]),
    ("row stride ignored", [("            float *row = x + t * ld + (int64_t)h * head_dim;\n            for (int i = 0;",
                             "            float *row = x + t * (int64_t)n_heads * head_dim + (int64_t)h * head_dim;\n            for (int i = 0;")]),
    # q/k-norm variant
    ("norm eps dropped", [("sqrt(ss / (double)head_dim + (double)eps)", "sqrt(ss / (double)head_dim)")]),
    ("norm mean over hd-1", [("sqrt(ss / (double)head_dim + (double)eps)", "sqrt(ss / (double)(head_dim - 1) + (double)eps)")]),
    ("norm without square root", [("1.0 / sqrt(ss / (double)head_dim + (double)eps)", "1.0 / (ss / (double)head_dim + (double)eps)")]),
    ("norm weight dropped", [("row[j] = (float)((double)row[j] * r * (double)w[j]);", "row[j] = (float)((double)row[j] * r);")]),
    ("norm stride ignored", [("            float *row = x + t * ld + (int64_t)h * head_dim;\n            double ss",
                              "            float *row = x + t * (int64_t)n_heads * head_dim + (int64_t)h * head_dim;\n            double ss")]),
    ("q norm uses k weight", [("oracle_rms_norm_heads(q, nt, ld_q, n_head, head_dim, wq, eps);", "oracle_rms_norm_heads(q, nt, ld_q, n_head, head_dim, wk, eps);")]),
    ("k not normalised", [("    oracle_rms_norm_heads(k, nt, ld_k, n_kv_head, head_dim, wk, eps);\n", "")]),
    ("v normalised too", [("    oracle_rms_norm_heads(k, nt, ld_k, n_kv_head, head_dim, wk, eps);\n",
                           "    oracle_rms_norm_heads(k, nt, ld_k, n_kv_head, head_dim, wk, eps);\n"
                           "    oracle_rms_norm_heads(v, nt, ld_v, n_kv_head, head_dim, wk, eps);\n")]),
    # norm after rope: the rope block is shared text in both chains, so a macro
    # expands to nothing in the plain chain and to the norm calls in the
    # q/k-norm chain (defined again just before that function)
    ("norm after rope", [("    oracle_rms_norm_heads(q, nt, ld_q, n_head, head_dim, wq, eps);\n"
                          "    oracle_rms_norm_heads(k, nt, ld_k, n_kv_head, head_dim, wk, eps);\n\n", ""),
                         ("#include <string.h>\n", "#include <string.h>\n#define NORM_AFTER_ROPE (void)0\n"),
                         ("int64_t oracle_qkv_norm_epilogue(",
                          "#undef NORM_AFTER_ROPE\n#define NORM_AFTER_ROPE "
                          "oracle_rms_norm_heads(q, nt, ld_q, n_head, head_dim, wq, eps); "
                          "oracle_rms_norm_heads(k, nt, ld_k, n_kv_head, head_dim, wk, eps)\n"
                          "int64_t oracle_qkv_norm_epilogue("),
                         ("    int64_t bad = oracle_store_rows(k, nt, ld_k, nkt, pos, slot, n_ctx,\n",
                          "    NORM_AFTER_ROPE;\n    int64_t bad = oracle_store_rows(k, nt, ld_k, nkt, pos, slot, n_ctx,\n")]),
    # rope variants
    ("interleaved reads the NeoX partner", [("float x1 = row[2 * i + 1];", "float x1 = row[i + half];")]),
    ("interleaved writes the NeoX partner", [("row[2 * i + 1] = (float)((double)x0 * s", "row[i + half] = (float)((double)x0 * s")]),
    ("frequency scale ignored", [("(float)((double)freq_scale * pow((double)theta, e))", "(float)(pow((double)theta, e))")]),
    ("frequency scale divides", [("(float)((double)freq_scale * pow((double)theta, e))", "(float)(pow((double)theta, e) / (double)freq_scale)")]),
    ("rope style ignored", [("    if (rope_style == 0) {", "    if (1) {")]),
    # projection
    ("projection weight transposed", [("oracle_bf16_to_double(w[n * hidden + k])", "oracle_bf16_to_double(w[k * n_out + n])")]),
    ("projection drops the last k", [("for (int64_t k = 0; k < hidden; ++k)\n                acc +=", "for (int64_t k = 0; k + 1 < hidden; ++k)\n                acc +=")]),
    ("projection bf16 decoded as low half", [("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b;")]),
    ("projection accumulates in f32", [("            double acc = 0.0;\n            for (int64_t k = 0; k < hidden; ++k)",
                                        "            float acc = 0.0f;\n            for (int64_t k = 0; k < hidden; ++k)")]),
    # 8-bit float weights
    ("e4m3 exponent bias 8", [("v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);")]),
    ("e4m3 subnormals read as normals", [("    if (e == 0)\n        v = ldexp((double)m, -9);", "    if (0)\n        v = ldexp((double)m, -9);")]),
    ("e4m3 sign ignored", [("    return sign ? -v : v;", "    return v;")]),
    ("e4m3 NaN pattern read as a number", [("    if (e == 15 && m == 7)\n        return NAN;", "    if (0)\n        return NAN;")]),
    ("fp8 row scale ignored", [("y[t * ld_y + n] = (float)((double)scale[n] * acc);", "y[t * ld_y + n] = (float)acc;")]),
    ("fp8 scale of the wrong row", [("y[t * ld_y + n] = (float)((double)scale[n] * acc);", "y[t * ld_y + n] = (float)((double)scale[0] * acc);")]),
    ("bias after norm", [("    if (bq)\n        oracle_add_bias(q, bq, nt, nqt, ld_q);\n", ""),
                         ("    oracle_rms_norm_heads(q, nt, ld_q, n_head, head_dim, wq, eps);\n",
                          "    oracle_rms_norm_heads(q, nt, ld_q, n_head, head_dim, wq, eps);\n"
                          "    if (bq)\n        oracle_add_bias(q, bq, nt, nqt, ld_q);\n")]),
]


def _pin_calls():
    """Every pin, with fixed parameters, as (name, zero-argument callable)."""
    return [
        ("inv_freq decimal 1e6/128", lambda: pins.test_inv_freq_matches_decimal(1.0e6, 128)),
        ("inv_freq decimal 1e4/64", lambda: pins.test_inv_freq_matches_decimal(1.0e4, 64)),
        ("inv_freq closed forms", pins.test_inv_freq_closed_forms),
        ("f16 golden table", pins.test_f16_golden_table),
        ("f16 vs numpy", pins.test_f16_matches_numpy_over_ranges),
        ("f16 nan", pins.test_f16_nan_stays_nan),
        ("hand-worked 1h4d", pins.test_handworked_1h4d),
        ("pos0 bias only (tiny)", lambda: pins.test_pos0_is_bias_only(wl.TINY_DECODE)),
        ("pos0 bias only (7B)", lambda: pins.test_pos0_is_bias_only(wl.DECODE_7B)),
        ("v bias only", pins.test_v_is_bias_only_at_any_position),
        ("norm preserved", lambda: pins.test_norm_preserved(wl.DECODE_14B)),
        ("complex multiply", pins.test_matches_complex_multiply_large_angles),
        ("decimal sin/cos", pins.test_cos_sin_match_decimal_at_large_positions),
        ("composition", pins.test_rotations_compose_additively),
        ("store brute force", pins.test_store_bruteforce_tiny),
        ("store f16 rows", pins.test_store_f16_rows_are_rne_of_outputs),
        ("slot rows and range", pins.test_slot_rows_and_range_errors),
        ("tokens independent", pins.test_tokens_are_independent),
        ("concat equals separate", pins.test_concat_rows_equal_separate_buffers),
        ("norm hand-worked", npins.test_handworked_3_4),
        ("norm constant vector", lambda: npins.test_constant_vector_closed_form(0.5, 1e-6)),
        ("norm tiny constant", lambda: npins.test_constant_vector_closed_form(1e-3, 1e-6)),
        ("norm scale invariance", npins.test_power_of_two_scale_invariance_is_exact),
        ("norm mean square", npins.test_mean_square_invariant),
        ("norm linalg", npins.test_matches_linalg_norm),
        ("norm heads independent", npins.test_heads_are_independent_and_stride_respected),
        ("variant pos0 (bias)", lambda: npins.test_variant_at_pos0_is_bias_then_norm(True)),
        ("variant pos0 (no bias)", lambda: npins.test_variant_at_pos0_is_bias_then_norm(False)),
        ("variant rotates after norm", npins.test_variant_rotates_after_norm),
        ("interleaved hand-worked", rpins.test_interleaved_handworked_1h4d),
        ("interleaved = permuted NeoX", lambda: rpins.test_interleaved_is_permuted_neox(64)),
        ("interleaved complex", rpins.test_interleaved_complex_multiply),
        ("scaled inv decimal", lambda: rpins.test_scaled_inv_freq_matches_decimal(0.25, 128)),
        ("scaled inv decimal 1/3", lambda: rpins.test_scaled_inv_freq_matches_decimal(1.0 / 3.0, 64)),
        ("scale 1 unscaled", rpins.test_scale_one_is_unscaled),
        ("scale = halved position (NeoX)", lambda: rpins.test_power_of_two_scale_equals_scaled_position(0)),
        ("scale = halved position (interleaved)", lambda: rpins.test_power_of_two_scale_equals_scaled_position(1)),
        ("chain style and scale", rpins.test_chain_style_and_scale_are_applied),
        ("projection exact rational", ppins.test_exact_rational_small),
        ("projection identity", ppins.test_identity_weights_copy_the_input),
        ("projection permutation", ppins.test_row_permutation_permutes_outputs),
        ("projection numpy", ppins.test_matches_numpy_float64_matmul),
        ("e4m3 table vs torch", fpins.test_code_table_matches_torch),
        ("e4m3 closed forms", fpins.test_code_table_closed_forms),
        ("fp8 projection exact rational", fpins.test_exact_rational_small),
        ("fp8 projection = bf16 of decoded", fpins.test_equals_bf16_projection_of_the_decoded_values),
        ("fp8 scale once per row", fpins.test_scale_applies_once_per_row),
        ("fp8 single codes", fpins.test_single_code_rows_decode_exactly),
    ]


def _build_mutant(edits, workdir):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor missing: {old!r}"
        src = src.replace(old, new)
    c = os.path.join(workdir, "mutant.c")
    so = os.path.join(workdir, "libmutant.so")
    open(c, "w").write(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-shared", "-fPIC", "-o", so, c, "-lm"])
    return so


def test_unmutated_copy_passes_every_pin(tmp_path):
    so = _build_mutant([], str(tmp_path))
    with oracle.using_library(so):
        for name, call in _pin_calls():
            call()


@pytest.mark.parametrize("name,edits", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, edits, tmp_path):
    so = _build_mutant(edits, str(tmp_path))
    caught = []
    with oracle.using_library(so):
        for pin, call in _pin_calls():
            try:
                call()
            except (AssertionError, ValueError):
                caught.append(pin)
    assert caught, f"planted mistake '{name}' survived every pin"
