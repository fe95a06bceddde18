"""Planted mistakes: each case copies oracle.c, plants one plausible mistake
(on the CPU, in a temporary directory), builds it and requires that at least
one pin fails on it.  This shows the pins are strong enough to catch a
dropped term, a wrong sign, a wrong index or a wrong rounding in the oracle."""
import os

import pytest

import oracle
from tests import pins

MUTANTS = {
    # encode: ties go to the lower code instead of the even one
    "tie_to_lower": ("else                code = (lo % 2 == 0) ? lo : hi;",
                     "else                code = lo;"),
    # encode: negative values that round to zero lose their sign
    "sign_from_compare": ("uint8_t sign = signbit(y) ? 0x80 : 0x00;",
                          "uint8_t sign = (y < 0) ? 0x80 : 0x00;"),
    # encode: no saturation, overflow takes the NaN code
    "no_saturation": ("if (m >= ORC_E4M3_MAX) return (uint8_t)(sign | 0x7E);",
                      "if (m >= 464.0) return (uint8_t)(sign | 0x7F);"),
    # decode: subnormal exponent off by one
    "subnormal_exp": ("if (e == 0) mag = ldexp((double)f, -9);",
                      "if (e == 0) mag = ldexp((double)f, -10);"),
    # scale: reciprocal-then-multiply instead of one division
    "scale_reciprocal": ("return (float)ORC_E4M3_MAX / d;",
                         "return (float)ORC_E4M3_MAX * (1.0f / d);"),
    # quantize: column copy uses the row scale
    "qt_row_scale": ("qt[c * rows + r] = orc_e4m3_encode(orc_bf16_to_f32(x[r * cols + c]) * s);",
                     "qt[c * rows + r] = orc_e4m3_encode(orc_bf16_to_f32(x[r * cols + c]) * scale[r]);"),
    # amax: absolute value dropped
    "amax_no_abs": ("float m = fabsf(v);", "float m = v;"),
    # GEMM: wrong operand index (first term of B taken from A's row)
    "gemm_operand": ("acc += val32[arow[t]] * val32[brow[t]];",
                     "acc += val32[arow[t]] * val32[arow[t]];"),
    # GEMM: one term dropped
    "gemm_drop_term": ("for (int64_t t = 0; t < k; t++)\n        acc +=",
                       "for (int64_t t = 1; t < k; t++)\n        acc +="),
    # epilogue: B's reciprocal taken from A's scale
    "epilogue_scale": ("float inv_b = 1.0f / sb;", "float inv_b = 1.0f / sa;"),
    # epilogue: bf16 rounding truncates
    "bf16_truncate": ("if (dd < du) return down;", "if (1) return down;"),
    # shard amax: first element skipped
    "amax_skip_first": ("for (int64_t i = 0; i < n; i++)\n        a = amax_update(",
                        "for (int64_t i = 1; i < n; i++)\n        a = amax_update("),
    # cast with a given scale: the scale is dropped
    "scaled_no_scale": ("float y = orc_bf16_to_f32(x[r * cols + c]) * s;",
                        "float y = orc_bf16_to_f32(x[r * cols + c]);"),
    # cast with a given scale: qt rows reversed
    "scaled_qt_index": ("uint8_t code = orc_e4m3_encode(y);\n            q[r * cols + c] = code;\n            qt[c * rows + r] = code;",
                        "uint8_t code = orc_e4m3_encode(y);\n            q[r * cols + c] = code;\n            qt[c * rows + (rows - 1 - r)] = code;"),
    # E5M2 decode: subnormal exponent off by one
    "e5m2_subnormal": ("else if (e == 0) mag = ldexp((double)f, -16);",
                       "else if (e == 0) mag = ldexp((double)f, -17);"),
    # E5M2 encode: overflow to infinity instead of saturation
    "e5m2_no_saturation": ("return (uint8_t)(sgn | 0x7B);", "return (uint8_t)(sgn | 0x7C);"),
    # E5M2 quantize: the E4M3 maximum in the scale
    "e5m2_scale_max": ("return (float)ORC_E5M2_MAX / d;", "return (float)ORC_E4M3_MAX / d;"),
    # mixed GEMM: B decoded with A's format
    "gemm_mixed_table": ("sum += ta[arow[t]] * tb[brow[t]];", "sum += ta[arow[t]] * ta[brow[t]];"),
    # fp32 GEMM: output stored transposed
    "gemm_f32_store": ("out[i * n + j] = gemm_element_f32(", "out[j * m + i] = gemm_element_f32("),
    # silu: wrong sign in the exponent
    "silu_exp_sign": ("return (float)(x / (1.0 + exp(-x)));", "return (float)(x / (1.0 + exp(x)));"),
    # silu': the (1 - sigma) factor dropped
    "dsilu_term": ("return (float)(sg * (1.0 + x * (1.0 - sg)));", "return (float)(sg * (1.0 + x));"),
    # SwiGLU forward: gate and value swapped
    "swiglu_swap": ("h[i] = orc_f32_to_bf16(orc_silu(av) * bv);",
                    "h[i] = orc_f32_to_bf16(orc_silu(bv) * av);"),
    # SwiGLU backward: the b factor of da dropped
    "swiglu_da_no_b": ("float gb = g * bv;", "float gb = g;"),
    # SwiGLU backward: db takes silu' instead of silu
    "swiglu_db_deriv": ("db[i] = orc_f32_to_bf16(g * orc_silu(av));",
                        "db[i] = orc_f32_to_bf16(g * orc_dsilu(av));"),
    # bf16 add: the second operand read from the first
    "add_operand": ("orc_f32_to_bf16(orc_bf16_to_f32(x[i]) + orc_bf16_to_f32(y[i]))",
                    "orc_f32_to_bf16(orc_bf16_to_f32(x[i]) + orc_bf16_to_f32(x[i]))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, "mutation site not found: %s" % name
    path = os.path.join(str(tmp_path), "oracle_%s.c" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(force=True, src=path, out=os.path.join(str(tmp_path), "lib%s.so" % name))
    mutant = oracle.Oracle(lib)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError as e:
            caught.append("%s: %s" % (check.__name__, e))
            break
    assert caught, "no pin caught mutant %s" % name
