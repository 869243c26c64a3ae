"""The pins have teeth: copies of the oracle with one plausible mistake planted
(a dropped term, a wrong sign or index, a transposed operand, the other rounding
rule) are compiled on the CPU and each must fail at least one pin."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ql_oracle.c")

# (name, text in ql_oracle.c, replacement)
MUTANTS = [
    ("round_half_away", "float r = nearbyintf(v[i] / s);\n        if (r > 127.0f)",
     "float r = roundf(v[i] / s);\n        if (r > 127.0f)"),
    ("reciprocal_multiply", "float r = nearbyintf(v[i] / s);\n        if (r > 127.0f)",
     "float r = nearbyintf(v[i] * (127.0f / (a > floor_a ? a : floor_a)));\n        if (r > 127.0f)"),
    ("int4_round_half_away", "float r = nearbyintf(v[i] / s);\n                if (r > 7.0f)",
     "float r = roundf(v[i] / s);\n                if (r > 7.0f)"),
    ("signed_absmax", "        float t = fabsf(v[i]);\n        if (t > a)\n            a = t;\n    }\n    const float floor_a = 1e-10f;",
     "        float t = v[i];\n        if (t > a)\n            a = t;\n    }\n    const float floor_a = 1e-10f;"),
    ("no_absmax_floor", "float s = (a > floor_a ? a : floor_a) / 127.0f;", "float s = a / 127.0f;"),
    ("scale_over_128", "float s = (a > floor_a ? a : floor_a) / 127.0f;", "float s = (a > floor_a ? a : floor_a) / 128.0f;"),
    ("gemm_transposed_w", "t += (int32_t)xq[m * K + k] * (int32_t)wq[n * K + k];",
     "t += (int32_t)xq[m * K + k] * (int32_t)wq[(k % N) * K + (n % K)];"),
    ("gemm_int16_accumulate", "t += (int32_t)xq[m * K + k] * (int32_t)wq[n * K + k];",
     "t = (int16_t)(t + (int32_t)xq[m * K + k] * (int32_t)wq[n * K + k]);"),
    ("epilogue_drops_bias", "                    y = y + bias[n];", "                    y = y;"),
    ("epilogue_wrong_scale_axis", "float y = t * x_scale[m];", "float y = t * x_scale[n % M];"),
    ("wonly_scale_row_major", "double s = group > 0 ? (double)scale[n * G + g] : (double)scale[n];",
     "double s = group > 0 ? (double)scale[g * N + n] : (double)scale[n];"),
    ("wonly_zero_sign", "acc += (double)x[m * K + k] * ((q - z) * s);", "acc += (double)x[m * K + k] * ((q + z) * s);"),
    ("int4_no_sign_extend", "return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    ("int4_nibble_order", "int nib = (int)((word >> (4 * (k % 8))) & 0xFu);",
     "int nib = (int)((word >> (4 * (7 - k % 8))) & 0xFu);"),
    ("w4a16_group_index", "scale16[n * G + k / group]", "scale16[n * G + (k % G)]"),
    ("int4_fp32_scale", "float s = oracle_f16_to_f32(h);", "float s = (a > floor_a ? a : floor_a) / 7.0f;"),
    ("int4_scale_over_8", "uint16_t h = oracle_f32_to_f16((a > floor_a ? a : floor_a) / 7.0f);",
     "uint16_t h = oracle_f32_to_f16((a > floor_a ? a : floor_a) / 8.0f);"),
    ("block_zero_sign", "float zf = nearbyintf(-mn / s);", "float zf = nearbyintf(mn / s);"),
    ("block_range_254", "float s = (mx - mn) / 255.0f;", "float s = (mx - mn) / 254.0f;"),
    ("f16_ties_away", "double r = nearbyint(ldexp(a, 10 - E));", "double r = round(ldexp(a, 10 - E));"),
    ("f16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("gelu_tanh_form", "y[i] = v * (0.5 * (1.0 + erf(v / sqrt(2.0))));",
     "y[i] = 0.5 * v * (1.0 + tanh(0.7978845608028654 * (v + 0.044715 * v * v * v)));"),
    ("gelu_no_sqrt2", "erf(v / sqrt(2.0))", "erf(v)"),
    ("silu_exp_sign", "y[i] = v / (1.0 + exp(-v));", "y[i] = v / (1.0 + exp(v));"),
    ("asym_zero_no_offset", "const float z = -lo / s - 128.0f;", "const float z = -lo / s;"),
    ("asym_zero_rounded", "const float z = -lo / s - 128.0f;", "const float z = nearbyintf(-lo / s) - 128.0f;"),
    ("asym_scale_254", "float s = (hi - lo) / 255.0f;", "float s = (hi - lo) / 254.0f;"),
    ("asym_min_is_max", "if (v[i] < lo)\n                lo = v[i];", "if (v[i] > lo)\n                lo = v[i];"),
    ("asym_clamp_127", "if (rq < -128.0f)\n                rq = -128.0f;", "if (rq < -127.0f)\n                rq = -127.0f;"),
    ("asym_no_scale_floor", "if (s < 1e-8f)\n            s = 1e-8f;", "if (s < 0.0f)\n            s = 1e-8f;"),
    ("asym_layer_zero_sign", "((double)xq[m * K + k] - (double)x_zero[m])", "((double)xq[m * K + k] + (double)x_zero[m])"),
    ("colsum_wrong_index", "t += wq[n * K + k];", "t += wq[(k % N) * K + (n % K)];"),
    ("e4m3_bias_8", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3_subnormal_exponent", "ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    ("e4m3_ties_up", "(d == bd && (c & 1) == 0 && (best & 1) == 1)", "(d == bd)"),
    ("e4m3_scale_127", "const float s = (a > 1e-10f ? a : 1e-10f) / 448.0f;",
     "const float s = (a > 1e-10f ? a : 1e-10f) / 127.0f;"),
    ("e4m3_gemm_abs_sum", "acc += p;", "acc += fabs(p);"),
    ("requant_half_away", "float r = nearbyintf(y[m * N + n] / sc);", "float r = roundf(y[m * N + n] / sc);"),
    ("requant_reciprocal", "float r = nearbyintf(y[m * N + n] / sc);", "float r = nearbyintf(y[m * N + n] * (1.0f / sc));"),
    ("requant_scale_by_row", "const float sc = s[scale_n == 1 ? 0 : n];", "const float sc = s[scale_n == 1 ? 0 : m % N];"),
    ("requant_clamp_128", "            if (r < -127.0f)\n                r = -127.0f;\n            q[m * N + n]",
     "            if (r < -128.0f)\n                r = -128.0f;\n            q[m * N + n]"),
    ("channel_scales_row_axis", "const float t = fabsf(y[m * N + n]);", "const float t = fabsf(y[(n * M + m) % (M * N)]);"),
    ("channel_scales_no_floor", "s[n] = (a > 1e-10f ? a : 1e-10f) / 127.0f;", "s[n] = a / 127.0f;"),
    ("asym_reciprocal", "const float t = v[i] / s + z;", "const float t = v[i] * (1.0f / s) + z;"),
    ("asym_zero_reciprocal", "const float z = -lo / s - 128.0f;", "const float z = -lo * (1.0f / s) - 128.0f;"),
    ("block_reciprocal", "int c = (int)nearbyintf(v[i] / s) + z;", "int c = (int)nearbyintf(v[i] * (1.0f / s)) + z;"),
    ("block_zero_reciprocal", "float zf = nearbyintf(-mn / s);", "float zf = nearbyintf(-mn * (1.0f / s));"),
    ("int4_reciprocal", "float r = nearbyintf(v[i] / s);\n                if (r > 7.0f)",
     "float r = nearbyintf(v[i] * (1.0f / s));\n                if (r > 7.0f)"),
    ("e4m3_reciprocal_448", "float t = v[i] / s;", "float t = v[i] * (448.0f / (a > 1e-10f ? a : 1e-10f));"),
    ("e4m3_reciprocal", "float t = v[i] / s;", "float t = v[i] * (1.0f / s);"),
    ("act_codes_swapped", "if (act == 1)\n            y[i] = v * (0.5", "if (act == 2)\n            y[i] = v * (0.5"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not found exactly once: " + name
    src = tmp_path / "ql_oracle.c"
    src.write_text(text.replace(old, new))
    hdr = os.path.join(os.path.dirname(SRC), "ql_oracle.h")
    (tmp_path / "ql_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(so), "-lm"])
    orc = oracle.Oracle(str(so))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, OverflowError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin catches the planted mistake " + name
