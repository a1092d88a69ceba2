"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them."""
import shutil

import pytest

import oracle
import oracle_pins

MUTATIONS = {
    "butterfly_sign": ("u[j + h] = a - c;", "u[j + h] = c - a;"),
    "stage_order_reversed": ("for (int h = 1; h < 256; h *= 2)", "for (int h = 128; h >= 1; h /= 2)"),
    "wrong_normalisation": ("u[j] = u[j] * 0.0625f;", "u[j] = u[j] * 0.125f;"),
    "scale_by_reciprocal": ("float s = amax / (float)qmax;", "float s = amax * (1.0f / (float)qmax);"),
    "round_half_away": ("float t = rintf(row[k] / s);", "float t = roundf(row[k] / s);"),
    "amax_without_abs": ("float a = fabsf(row[k]);", "float a = row[k];"),
    "gemm_output_transposed": ("acc[m * N + n] = (int32_t)s;", "acc[n * M + m] = (int32_t)s;"),
    "gemm_row_offset_wrong": ("s += (int64_t)a[m * lda + k] * (int64_t)w[n * ldw + k];", "s += (int64_t)a[m * lda + k] * (int64_t)w[n * ldw + (k + 1) % K];"),
    "epilogue_scale_order": ("t = t * sx;\n    t = t * sw;", "t = t * (sx * sw);"),
    "epilogue_bias_dropped": ("if (bias) t = t + bf16_bits_to_float(bias[n]);", "(void)bias; (void)n;"),
    "bf16_round_half_up": ("return (uint16_t)((u + 0x7fffu + lsb) >> 16);", "return (uint16_t)((u + 0x8000u + 0 * lsb) >> 16);"),
    "dequant_divides": ("float v = (float)q[m * ldq + k] * s;", "float v = (float)q[m * ldq + k] / s;"),
    "int4_nibbles_swapped": ("packed[r * (K / 2) + i] = (uint8_t)(lo | (hi << 4));", "packed[r * (K / 2) + i] = (uint8_t)(hi | (lo << 4));"),
    "rotation_skips_last_block": ("for (int64_t b = 0; b < K; b += 256)", "for (int64_t b = 0; b + 256 < K; b += 256)"),
    "bf16_widen_wrong_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "tensorwise_first_row_only": ("for (int64_t r = 0; r < M; r++)", "for (int64_t r = 0; r < 1; r++)"),
    "tensorwise_qmax_off_by_one": ("const float ts = tmax / (float)qmax;", "const float ts = tmax / (float)(qmax + 1);"),
    "gelu_cubic_coefficient": ("(x + 0.044715L * x * x * x)", "(x + 0.04715L * x * x * x)"),
    "silu_exponent_sign": ("return x / (1.0L + expl(-x));", "return x / (1.0L + expl(x));"),
    "gelu_erf_argument_sign": ("erfcl(-x / sqrtl(2.0L))", "erfcl(x / sqrtl(2.0L))"),
    "act_rounding_one_bit_short": ("round_to_grid(a, 7, -126)", "round_to_grid(a, 6, -126)"),
    "act_fp16_no_subnormals": ("round_to_grid(a, 10, -14)", "round_to_grid(a, 10, -24)"),
    "relu_passes_negatives": ("case ORACLE_ACT_RELU: return x > 0.0L ? x : 0.0L;", "case ORACLE_ACT_RELU: return x;"),
    "attention_scale_missing": ("(double)sk[kr] * scale;", "(double)sk[kr];"),
    "attention_value_scale_dropped": ("num += sc[j] * ((double)sv[vr] * (double)vc[vr * D + d]);",
                                      "num += sc[j] * (double)vc[vr * D + d];"),
    "attention_not_normalised": ("out[qi * D + d] = num / den;", "out[qi * D + d] = num;"),
    "attention_keys_of_head0": ("const int64_t kr = bh * Lk + j;", "const int64_t kr = j;"),
    "attention_probs_not_normalised": ("for (int64_t j = 0; j < Lk; j++) pr[j] = pr[j] / den;",
                                       "for (int64_t j = 0; j < Lk; j++) pr[j] = pr[j] / (den + 1.0);"),
    "attention_key_scale_of_query": ("(double)sq[qi] * (double)sk[kr]", "(double)sq[qi] * (double)sq[qi]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTATIONS[name]
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(path), str(tmp_path / f"lib_{name}.so"))
    O = oracle.Oracle(lib)
    caught = None
    for check in oracle_pins.CHECKS:          # quick checks first; stop at the first that fails
        try:
            check(O)
        except (AssertionError, OverflowError, ValueError, RuntimeError):
            caught = check.__name__
            break
    assert caught, f"mutation {name} not caught by any pin"
