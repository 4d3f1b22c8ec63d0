"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of oracle/glu_oracle.c (a dropped term,
a wrong sign, a swapped or transposed operand, a wrong tie rule, a wrong constant),
builds it, routes the oracle module to it and runs a few pin tests.  At least one pin
must fail for every mutant; the real oracle is untouched.
"""
import os
import tempfile

import pytest

import oracle
from oracle import build as obuild
import test_oracle_formats as tf
import test_oracle_glu as tg
import test_oracle_quant as tq

S, G, E, R = oracle.SWIGLU, oracle.GEGLU_TANH, oracle.GEGLU_ERF, oracle.RELU2

# (name, text to find, replacement, pins that should notice)
MUTANTS = [
    ("gelu drops x^3", "GELU_K0 * (x + GELU_K1 * x * x * x)", "GELU_K0 * (x)",
     [lambda: tg.test_act_against_mpmath(G)]),
    ("silu' sign", "logistic(x) * (1.0 + x * logistic(-x))", "logistic(x) * (1.0 - x * logistic(-x))",
     [lambda: tg.test_act_grad_against_mpmath(S)]),
    ("gelu' drops the 3", "3.0 * GELU_K1", "GELU_K1",
     [lambda: tg.test_act_grad_against_mpmath(G)]),
    ("gelu' drops a factor", "(1.0 + x * one_minus_t * GELU_K0", "(1.0 + x * GELU_K0",
     [lambda: tg.test_act_grad_against_autograd(G)]),
    ("gelu' as a sum of terms", "return 0.5 * one_plus_t *\n         (1.0 + x * one_minus_t",
     "return 0.5 * one_plus_t + 0.5 * one_plus_t *\n         (x * one_minus_t",
     [lambda: tg.test_act_and_grad_negative_in_the_tail(G)]),
    ("erf-GELU' loses the sign of zero", "(d == 0.0 && x < 0.0 && isfinite(x)) ? -0.0 : d", "d",
     [lambda: tg.test_act_and_grad_negative_in_the_tail(E)]),
    ("erf-GELU CDF sign", "0.5 * erfc(-x * SQRT1_2)", "0.5 * erfc(x * SQRT1_2)",
     [lambda: tg.test_act_against_mpmath(E)]),
    ("erf-GELU' drops x", "normal_cdf(x) + x * normal_pdf(x)", "normal_cdf(x) + normal_pdf(x)",
     [lambda: tg.test_act_grad_against_autograd(E)]),
    ("erf-GELU density exponent", "exp(-0.5 * x * x)", "exp(-x * x)",
     [lambda: tg.test_act_grad_against_mpmath(E)]),
    ("relu2' drops the 2", "return 2.0 * relu(x);", "return relu(x);",
     [lambda: tg.test_act_grad_against_autograd(R)]),
    ("relu2 is plain relu", "return relu(x) * relu(x);", "return relu(x);",
     [tg.test_relu2_glu_is_exact]),
    ("relu drops NaN", "(x <= 0.0 ? 0.0 : x)", "0.0", [tg.test_act_special_values]),
    ("ties away from zero", "return (lo % 2 == 0) ? lo : hi;", "return hi;",
     [tf.test_e4m3_golden, tf.test_e2m1_golden, tf.test_bf16_overflow_and_specials]),
    ("RCEIL on equality", "ldexp(448.0, e) < amax", "ldexp(448.0, e) <= amax",
     [tf.test_rceil_golden]),
    ("RCEIL rounds down", "while (e < 127 && ldexp(448.0, e) < amax) e++;",
     "while (e < 127 && ldexp(448.0, e + 1) < amax) e++;", [tf.test_rceil_golden]),
    ("colwise scales transposed", "&s_col[sf_pos(j, b, M / 32, swz)]", "&s_col[sf_pos(b, j, N, swz)]",
     [tq.test_mx_colwise_is_rowwise_of_transpose]),
    ("swizzled MX scales unpadded", "swizzled ? orc_sf128x4_offset(r, c, (nb + 3) / 4 * 4)",
     "swizzled ? orc_sf128x4_offset(r, c, nb)",
     [tq.test_mx_swizzled_scales_equal_rowmajor_after_unswizzle]),
    ("colwise codes transposed", "memcpy(&q_col[j * M + 32 * b], c, 32);",
     "for (int i = 0; i < 32; i++) q_col[(32 * b + i) * N + j] = c[i];",
     [tq.test_mx_golden_blocks_rowwise_and_colwise]),
    ("nibble order", "(c[2 * k] | (c[2 * k + 1] << 4))", "(c[2 * k + 1] | (c[2 * k] << 4))",
     [tq.test_nv_golden_blocks]),
    ("gate and up swapped", "*g = orc_bf16_to_f64(gate[m * ld + j]);\n    *u = orc_bf16_to_f64(up[m * ld + j]);",
     "*g = orc_bf16_to_f64(up[m * ld + j]);\n    *u = orc_bf16_to_f64(gate[m * ld + j]);",
     [lambda: tg.test_glu_fwd_matches_float64_reference(S)]),
    ("da drops up", "d * u * orc_act_grad(act, g)", "d * orc_act_grad(act, g)",
     [lambda: tg.test_glu_bwd_matches_autograd(S)]),
    ("paired columns swapped", "*g = orc_bf16_to_f64(gate[m * ld + 2 * j]);", "*g = orc_bf16_to_f64(gate[m * ld + 2 * j + 1]);",
     [tg.test_layouts_agree]),
    ("NV backward halves swapped",
     "orc_glu_bwd(act, ORC_SPLIT, M, N, gate, up, ld, dh, lddh, d, d + N, 2 * N);\n  float* x = widen_bf16(d, M * 2 * N);\n  free(d);\n  if (!x) return -1;\n  orc_quant_nvfp4",
     "orc_glu_bwd(act, ORC_SPLIT, M, N, gate, up, ld, dh, lddh, d + N, d, 2 * N);\n  float* x = widen_bf16(d, M * 2 * N);\n  free(d);\n  if (!x) return -1;\n  orc_quant_nvfp4",
     [tq.test_nv_backward_is_da_then_db]),
    ("NV global scale drops the 6", "const float s = 2688.0f / amax;", "const float s = 448.0f / amax;",
     [tq.test_nv_global_scale_closed_forms]),
    ("NV two-level block scale ignores the 6", "const float d = amax * k;", "const float d = amax * s;",
     [tq.test_nv_gs_blocks_against_brute_force]),
    ("NV two-level codes inverted", "const float r = S == 0.0f ? 0.0f : s / S;",
     "const float r = S == 0.0f ? 0.0f : S / s;", [tq.test_nv_gs_blocks_against_brute_force]),
    ("GEMM scale bias", "ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 126)",
     [tq.test_mx_gemm_closed_forms]),
    ("GEMM epilogue gate column off by one", "return w_layout == ORC_PAIRED ? 2 * j : j;",
     "return w_layout == ORC_PAIRED ? 2 * j : j + 1;", [tq.test_glu_gemm_is_glu_of_the_gemm]),
    ("GEMM interleaved W: gate and up rows swapped", "return w_layout == ORC_PAIRED ? 2 * j + 1 : N + j;",
     "return w_layout == ORC_PAIRED ? 2 * j : N + j;", [tq.test_glu_gemm_interleaved_w_rows]),
    ("E2M1 operand row pitch", "rb = fmt == ORC_FMT_E2M1 ? K / 2 : K;", "rb = K;",
     [tq.test_mx_gemm_e2m1_matches_numpy_on_dequantized_operands]),
    ("E2M1 operand read as E4M3", "if (fmt == ORC_FMT_E2M1) {", "if (0) {",
     [tq.test_mx_gemm_e2m1_closed_forms]),
    ("GEMM drops a block's scale", "acc += blk * sx * sw;", "acc += blk * sx;",
     [tq.test_mx_gemm_matches_numpy_on_dequantized_operands]),
    ("NV scale divisor", "amax / 6.0", "amax / 4.0", [tq.test_nv_golden_blocks]),
    ("MX scale direction", "ldexp(v[i], -e)", "ldexp(v[i], e)", [tq.test_mx_golden_blocks_rowwise_and_colwise]),
    ("bf16 subnormal exponent", "ldexp((double)m, -133)", "ldexp((double)m, -134)",
     [tf.test_bf16_overflow_and_specials]),
    ("E2M1 saturation", "nearest_code(fabs(y), e2m1_mag, 7)", "nearest_code(fabs(y), e2m1_mag, 6)",
     [tf.test_e2m1_golden]),
    ("E4M3 subnormal step", "ldexp((double)m, -9)", "ldexp((double)m, -10)", [tf.test_e4m3_decode_matches_torch]),
    ("non-finite blocks ignored", "if (!isfinite(v[i])) finite = 0;", "if (0) finite = 0;",
     [tq.test_mx_nonfinite_block_reading]),
    ("128x4 row interleave", "(r % 32) * 16 +\n         ((r % 128) / 32) * 4", "(r % 32) * 4 +\n         ((r % 128) / 32) * 16",
     [tq.test_sf128x4_layout_is_zero_padded_permutation]),
]


def _fails(pin) -> bool:
    try:
        pin()
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name,find,repl,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, find, repl, pins):
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(find) >= 1, f"mutation site not found: {name}"
    with tempfile.TemporaryDirectory() as d:
        msrc = os.path.join(d, "mutant.c")
        with open(msrc, "w") as f:
            f.write(src.replace(find, repl))
        lib = obuild.build(src=msrc, lib=os.path.join(d, "libmutant.so"))
        with oracle.use_library(lib):
            assert any(_fails(p) for p in pins), f"no pin noticed: {name}"
    # the real oracle still passes the same pins
    for p in pins:
        p()
