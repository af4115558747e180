"""CPU: the oracle against its pins, and planted mistakes against the pins.

Each mutant below is a plausible slip in the oracle (a dropped term, an
inverted direction, a wrong rounding mode, a wrong index...). The source is
patched in a temporary directory, compiled, loaded, and every pin is run; at
least one pin must fail for each mutant, or the pins would not be able to
catch that mistake in the real oracle.
"""
import os
import subprocess

import pytest

from oracle import oracle as oracle_mod
from tests import oracle_pins

ORACLE = oracle_mod.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ORACLE)


MUTANTS = {
    "inverted_direction": ("s[j] = (float)(num / den);", "s[j] = (float)(den / num);"),
    "dropped_weight_term": ("double den = pow((double)w, 1.0 - alpha);", "double den = 1.0;"),
    "round_half_away": ("float r = rintf(v);", "float r = roundf(v);"),
    "truncate": ("float r = rintf(v);", "float r = truncf(v);"),
    "clamp_minus_128": ("if (r < -SQO_QMAX) r = -SQO_QMAX;", "if (r < -128.0f) r = -128.0f;"),
    "max_without_abs": ("float v = fabsf(elem(x, xtype, t * k + j));", "float v = elem(x, xtype, t * k + j);"),
    "act_scale_over_128": ("return mx / SQO_QMAX;", "return mx / 128.0f;"),
    "act_scale_ignores_s": ("float v = a * inv_s[j];", "float v = a;"),
    "weight_divided_by_s": ("row[j] = elem(w, wtype, r * k + j) * s[j];",
                            "row[j] = elem(w, wtype, r * k + j) / s[j];"),
    "act_multiplied_by_s": ("float smoothed = elem(x, xtype, r * k + j) * inv_s[j];",
                            "float smoothed = elem(x, xtype, r * k + j) / inv_s[j];"),
    "quantize_before_smoothing": ("xq[r * k + j] = quantize_scaled(smoothed * inv_a);",
                                  "xq[r * k + j] = quantize_scaled(elem(x, xtype, r * k + j) * inv_a); (void)smoothed;"),
    "dequant_row_scale": ("float scale = act_scale * w_scale[c];", "float scale = act_scale * w_scale[r % n];"),
    "gemm_reversed_k": ("(int64_t)wq[c * k + j];", "(int64_t)wq[c * k + (k - 1 - j)];"),
    "no_row_floor": ("if (mx < SQO_FLOOR) mx = SQO_FLOOR;", ""),
    "sse_abs": ("acc += d * d;", "acc += fabs(d);"),
    "argmax_not_argmin": ("if (mse[i] < mse[best]) best = i;", "if (mse[i] > mse[best]) best = i;"),
    "weight_scale_over_128": ("float ws = mx / SQO_QMAX;", "float ws = mx / 128.0f;"),
    "ref_gemm_float_accum": ("double sum = 0.0;\n        for (int64_t j = 0; j < k; ++j)\n            sum += (double)elem(x",
                             "float sum = 0.0f;\n        for (int64_t j = 0; j < k; ++j)\n            sum += (float)elem(x"),
    "dynamic_scale_half_channels": ("float a = sqo_act_scale(live, inv_s, k);",
                                    "float a = sqo_act_scale(live, inv_s, k / 2);"),
    "dynamic_scale_unsmoothed": ("float a = sqo_act_scale(live, inv_s, k);",
                                 "float* one = (float*)malloc((size_t)k * sizeof(float));\n    for (int64_t j = 0; j < k; ++j) one[j] = 1.0f;\n    float a = sqo_act_scale(live, one, k);\n    free(one);"),
    "sample_max_runs_on": ("for (int64_t b = 0; b < samples; ++b) {\n            float mx = 0.0f;",
                           "float mx = 0.0f;\n        for (int64_t b = 0; b < samples; ++b) {"),
    "mean_off_by_one": ("act_max[j] = (float)(sum[j] / (double)count);",
                        "act_max[j] = (float)(sum[j] / (double)(count + 1));"),
    "percentile_rank_floor": ("int64_t rank = (int64_t)ceil(q * (double)rows);",
                              "int64_t rank = (int64_t)floor(q * (double)rows);"),
    "percentile_descending": ("return (x > y) - (x < y);", "return (x < y) - (x > y);"),
    "rms_sum_not_mean": ("r[t] = (float)(1.0 / sqrt(ss / (double)k + (double)eps));",
                         "r[t] = (float)(1.0 / sqrt(ss + (double)eps));"),
    "rms_eps_outside": ("r[t] = (float)(1.0 / sqrt(ss / (double)k + (double)eps));",
                        "r[t] = (float)(1.0 / sqrt(ss / (double)k) + (double)eps);"),
    "rms_no_sqrt": ("r[t] = (float)(1.0 / sqrt(ss / (double)k + (double)eps));",
                    "r[t] = (float)(1.0 / (ss / (double)k + (double)eps));"),
    "fold_multiplies_s": ("gamma_folded[j] = gamma[j] * inv_s[j];", "gamma_folded[j] = gamma[j] / inv_s[j];"),
    "norm_quant_drops_gamma": ("float smoothed = (elem(h, htype, t * k + j) * r[t]) * gamma_folded[j];",
                               "float smoothed = elem(h, htype, t * k + j) * r[t]; (void)gamma_folded;"),
    "e4m3_truncates": ("float q = rintf(ldexpf(a, 3 - E));", "float q = truncf(ldexpf(a, 3 - E));"),
    "e4m3_bias_8": ("return sign | (uint8_t)(((E + 7) << 3) | ((int)q - 8));",
                    "return sign | (uint8_t)(((E + 8) << 3) | ((int)q - 8));"),
    "e4m3_subnormal_step": ("float q = rintf(ldexpf(a, 9));", "float q = rintf(ldexpf(a, 10));"),
    "fp8_weight_scale_127": ("float ws = mx / SQO_FP8_MAX;", "float ws = mx / 127.0f;"),
    "fp8_act_scale_ignores_s": ("float v = inv_s[j] * a;", "float v = a;"),
    "fp8_gemm_drops_sign": ("double p = (double)sqo_e4m3_decode(xq[r * k + j]) * (double)sqo_e4m3_decode(wq[c * k + j]);",
                            "double p = fabs((double)sqo_e4m3_decode(xq[r * k + j])) * (double)sqo_e4m3_decode(wq[c * k + j]);"),
    "dequant_f32_act_scale_only": ("float merged = w_scale[c] * act_scale;", "float merged = act_scale;"),
    "norm_quant_drops_r": ("float smoothed = (elem(h, htype, t * k + j) * r[t]) * gamma_folded[j];",
                           "float smoothed = elem(h, htype, t * k + j) * gamma_folded[j];"),
    # fp16 scale storage (O25-O29)
    "f16_truncates": ("float q = rintf(ldexpf(a, 10 - E));", "float q = truncf(ldexpf(a, 10 - E));"),
    "f16_bias_16": ("return sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024));",
                    "return sign | (uint16_t)(((E + 16) << 10) | ((int)q - 1024));"),
    "f16_subnormal_step": ("float q = rintf(ldexpf(a, 24));", "float q = rintf(ldexpf(a, 23));"),
    "f16_scale_no_floor": ("if (v < SQO_F16_MIN) v = SQO_F16_MIN;", ""),
    "f16_scale_overflows": ("if (v > SQO_F16_MAX) v = SQO_F16_MAX;", ""),
    "f16_act_scale_from_unrounded_s": ("float inv = 1.0f / sqo_f16_decode(s16[j]);", "float inv = 1.0f / s;"),
    "f16_weight_codes_unrounded_scale": ("float inv_ws = 1.0f / sqo_f16_decode(w_scale16[r]);",
                                         "float inv_ws = 1.0f / ((mx < SQO_FLOOR ? SQO_FLOOR : mx) / SQO_QMAX);"),
    "f16_fold_reads_s_as_bf16": ("row[j] = elem(w, wtype, r * k + j) * sqo_f16_decode(s16[j]);",
                                 "row[j] = elem(w, wtype, r * k + j) * bf16_bits_to_float(s16[j]);"),
    "f16_act_codes_unrounded_act_scale": ("float inv_a = 1.0f / sqo_f16_decode(act_scale16);\n    float* inv_s",
                                          "float inv_a = 1.0f / sqo_f16_decode(act_scale16 + 1);\n    float* inv_s"),
    "f16_dequant_drops_weight_scale": ("float merged = a * sqo_f16_decode(w_scale16[c]);", "float merged = a;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle_mod.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    (tmp_path / "sq_oracle.h").write_text(open(os.path.join(oracle_mod.HERE, "sq_oracle.h")).read())
    (tmp_path / "sq_oracle.c").write_text(src.replace(old, new))
    lib = oracle_mod.build(str(tmp_path / "sq_oracle.c"), str(tmp_path / f"libmut_{name}.so"))
    o = oracle_mod.Oracle(oracle_mod.load(lib))
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
