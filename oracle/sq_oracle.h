/*
 * sq_oracle.h -- plain CPU reference for the SmoothQuant W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this; it exists so the GPU library can be checked against a slow,
 * obviously correct definition written from the pages' text. It shares no
 * code, header, table or constant with the GPU library.
 *
 * Sources (cited by page and section; "kwkr.cn blog" is the Chinese
 * engineering write-up on SmoothQuant W8A8 at kwkr.cn/news/621929, "ADR-010"
 * is "010. SmoothQuant Integration" on blog.yoooo.fun, "pwwt.cn" is
 * "SmoothQuant技术解析：LLM模型INT8无损量化实践", "tbr8.org" is the page on
 * activation outliers and SmoothQuant with the PyTorch example):
 *   - calibration statistics:      kwkr.cn blog §3.1; ADR-010 "Layer 2" (add_batch)
 *   - smoothing factor s_j:        kwkr.cn blog §2.2; ADR-010 "Context" item 1
 *   - weight fold + per-row int8:  kwkr.cn blog §3.2, §3.3; ADR-010 "Context" items 2-3
 *   - activation x/s + per-tensor: ADR-010 "Key design" items 1, 4, 5; kwkr.cn blog §3.2
 *   - symmetric quantizer:         kwkr.cn blog §1.2
 *   - int8 GEMM + merged scales:   pwwt.cn §3.1 (quantized_matmul_kernel stub)
 *   - alpha grid search:           ADR-010 "Key design" item 2
 *   - dynamic mode:                pwwt.cn §2.3 (static vs dynamic scales)
 *   - robust calibration:          kwkr.cn blog §3.1 (percentile, mean of maxima)
 *   - 1/s folded into the norm:    kwkr.cn blog §2.3 and §3.2 (gamma of the
 *                                  preceding norm absorbs 1/s)
 *   - FP8 after smoothing:         aiunderstanding.org, "SmoothQuant 和激活量化"
 *                                  (the section on where smoothing goes next:
 *                                  INT8 and FP8 serving)
 *
 * Conventions: X[m,k] and W[n,k] are row-major with k contiguous; column j is
 * input channel j. Every floating-point step is one IEEE fp32 operation with
 * round-to-nearest-even and no fused multiply-add (built with
 * -ffp-contract=off), except where fp64 is stated. bf16 inputs are widened to
 * fp32 exactly.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py.
 */
#ifndef SQ_ORACLE_H
#define SQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of floating-point buffers */
enum { SQO_F32 = 0, SQO_BF16 = 1 };

/* Number of OpenMP threads the oracle's outer loops use. */
int sqo_num_threads(void);

/* Set that number for later calls from the calling thread (n < 1 means 1).
 * Results do not depend on it: the parallel loops run over independent rows
 * or columns, and per-row partial sums are added in row order afterwards. */
void sqo_set_num_threads(int n);

/* O1/O2: absmax[j] = max(absmax_in[j] if accumulate else 0, max_t |x[t,j]|). */
void sqo_calib_absmax(const void* x, int xtype, int64_t rows, int64_t k,
                      float* absmax, int accumulate);

/* O6 alone: mx = max_j fl(max(act_max[j],1e-5) * inv_s[j]); returns fl(mx/127). */
float sqo_act_scale(const float* act_max, const float* inv_s, int64_t k);

/* O3-O6: s, inv_s (length k) and the per-tensor activation scale. */
void sqo_smooth_factors(const float* act_max, const float* w_max, int64_t k,
                        double alpha, float* s, float* inv_s, float* act_scale);

/* O7: W' = W*diag(s) (per column j), per-row symmetric int8. */
void sqo_quant_weight(const void* w, int wtype, int64_t n, int64_t k,
                      const float* s, int8_t* wq, float* w_scale);

/* O8: xq = clamp(rne(fl(fl(x*inv_s[j]) * fl(1/act_scale))), -127, 127). */
void sqo_quant_act(const void* x, int xtype, int64_t m, int64_t k,
                   const float* inv_s, float act_scale, int8_t* xq);

/* O9: acc[m,n] = sum_j xq[m,j]*wq[n,j], exact in integers. */
void sqo_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n,
                  int64_t k, int32_t* acc);

/* O10: y[m,n] = fl(fl(float(acc)) * fl(act_scale*w_scale[n])); ytype F32 or
 * BF16 (bf16 = round-to-nearest-even of the fp32 value). */
void sqo_dequant(const int32_t* acc, int64_t m, int64_t n, float act_scale,
                 const float* w_scale, int ytype, void* y);

/* Reference product: yref[m,n] = (float) sum_j (double)x[m,j]*(double)w[n,j],
 * summed in ascending j. */
void sqo_ref_gemm(const void* x, int xtype, const void* w, int wtype,
                  int64_t m, int64_t n, int64_t k, float* yref);

/* Squared error: sum over (m,n) of ((double)y - (double)yref)^2, rows summed
 * in ascending order. */
double sqo_sse(const float* y, const float* yref, int64_t m, int64_t n);

/* O11: alpha grid search. x_batches: nb host pointers, each [rows,k]. Writes
 * mse[na] and returns the first index attaining the minimum. */
int sqo_alpha_search(const void* const* x_batches, int xtype, int nb,
                     int64_t rows, int64_t k, const void* w, int wtype,
                     int64_t n, const double* alphas, int na, double* mse);

/* O13: dynamic mode. The smoothing factors stay the offline ones; the
 * per-tensor activation scale is recomputed from the live batch with the O6
 * closed form: live[j] = max_t |x[t,j]|, a = O6(live, inv_s), then O8 with a.
 * Writes xq and a. */
void sqo_dynamic_quant_act(const void* x, int xtype, int64_t m, int64_t k,
                           const float* inv_s, int8_t* xq, float* act_scale);

/* O14: mean of per-sample maxima. x holds `samples` consecutive samples of
 * rows_per_sample rows each; sum[j] += (double) max_{t in sample} |x[t,j]|,
 * the samples added in ascending order (a running sum across calls). */
void sqo_calib_sample_max_sum(const void* x, int xtype, int64_t samples,
                              int64_t rows_per_sample, int64_t k, double* sum);

/* O14 (end): act_max[j] = (float)(sum[j] / (double)count). */
void sqo_calib_mean_finalize(const double* sum, int64_t count, int64_t k,
                             float* act_max);

/* O15: nearest-rank percentile of |x[:,j]| over the rows: the rank-th
 * smallest magnitude, rank = sqo_percentile_rank(q, rows). */
int64_t sqo_percentile_rank(double q, int64_t rows);
void sqo_calib_percentile(const void* x, int xtype, int64_t rows, int64_t k,
                          double q, float* act_max);

/* O16: RMSNorm (the norm in front of every projection of a Llama block).
 * r[t] = (float)(1 / sqrt(sum_j h[t,j]^2 / k + eps)) evaluated in fp64 with
 * the squares summed in ascending j and rounded once. */
void sqo_rms_inv(const void* h, int htype, int64_t m, int64_t k, float eps,
                 float* r);

/* O16 (apply): y[t,j] = fl(fl(h[t,j] * r[t]) * gamma[j]), fp32 or bf16 (RNE). */
void sqo_rmsnorm_apply(const void* h, int htype, int64_t m, int64_t k,
                       const float* r, const float* gamma, int ytype, void* y);

/* O17: 1/s folded into the norm weight: gamma_folded[j] = fl(gamma[j] * inv_s[j]). */
void sqo_fold_norm_weight(const float* gamma, const float* inv_s, int64_t k,
                          float* gamma_folded);

/* O18: the norm with the folded weight feeding the per-tensor quantizer
 * directly: xq[t,j] = q(fl(fl(fl(h[t,j] * r[t]) * gamma_folded[j]) * fl(1/a))),
 * q = round half to even, clamp to [-127, 127]. Given r (from O16). */
void sqo_norm_quant_apply(const void* h, int htype, int64_t m, int64_t k,
                          const float* r, const float* gamma_folded,
                          float act_scale, int8_t* xq);

/* O19: OCP FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, largest finite 448): round-to-nearest-even encoding of a
 * finite fp32 value; magnitudes that would round past 448 saturate to 448.
 * Decoding is exact. */
uint8_t sqo_e4m3_encode(float v);
float sqo_e4m3_decode(uint8_t b);

/* O20: the FP8 variant of O7: W' = W*diag(s); w_scale[r] = fl(max(max_j
 * |W'[r,j]|, 1e-5) / 448); wq[r,j] = e4m3(fl(W'[r,j] * fl(1/w_scale[r]))). */
void sqo_quant_weight_fp8(const void* w, int wtype, int64_t n, int64_t k,
                          const float* s, uint8_t* wq, float* w_scale);

/* O21: the FP8 variant of O6: fl(max_j fl(max(act_max[j],1e-5)*inv_s[j]) / 448). */
float sqo_act_scale_fp8(const float* act_max, const float* inv_s, int64_t k);

/* O22: the FP8 variant of O8: xq = e4m3(fl(fl(x*inv_s[j]) * fl(1/act_scale))). */
void sqo_quant_act_fp8(const void* x, int xtype, int64_t m, int64_t k,
                       const float* inv_s, float act_scale, uint8_t* xq);

/* O23: acc[r,c] = sum_j decode(xq[r,j]) * decode(wq[c,j]) in fp64 (exact for
 * k below 2^16: each product has at most 8 significant bits and lies in
 * [2^-18, 2^18)); then y = fl(fl(acc) * fl(act_scale * w_scale[c])), fp32 or
 * bf16 (RNE), and the fp64 sums of |products| (for error bounds) in absacc. */
void sqo_gemm_fp8(const uint8_t* xq, const uint8_t* wq, int64_t m, int64_t n,
                  int64_t k, float act_scale, const float* w_scale, int ytype,
                  void* y, double* acc, double* absacc);

/* O24: O10 for an fp32 accumulator (the FP8 product's): y = fl(acc *
 * fl(act_scale * w_scale[n])), fp32 or bf16 (RNE). */
void sqo_dequant_f32(const float* acc, int64_t m, int64_t n, float act_scale,
                     const float* w_scale, int ytype, void* y);

/* O25: IEEE binary16 encode (round to nearest even, overflow to infinity)
 * and decode, for the fp16 scale storage of ADR-010 "Consequences";
 * sqo_scale_f16 keeps a positive scale inside [2^-24, 65504] first. */
uint16_t sqo_f16_encode(float v);
float sqo_f16_decode(uint16_t h);
uint16_t sqo_scale_f16(float v);
void sqo_f16_encode_array(const float* v, int64_t n, uint16_t* out);
void sqo_f16_decode_array(const uint16_t* h, int64_t n, float* out);

/* O26: s16[j] = scale_f16(s_j) with s_j as O4; act_scale16 =
 * scale_f16(fl(max_j fl(max(act_max[j],1e-5) * fl(1/dec(s16[j]))) / 127)). */
void sqo_smooth_factors_h(const float* act_max, const float* w_max, int64_t k,
                          double alpha, uint16_t* s16, uint16_t* act_scale16);

/* O27: W' = fl(W * dec(s16)); w_scale16[r] = scale_f16(fl(max(max_j |W'|,
 * 1e-5) / 127)); wq = clamp(rne(fl(W' * fl(1/dec(w_scale16[r])))), +-127). */
void sqo_quant_weight_h(const void* w, int wtype, int64_t n, int64_t k,
                        const uint16_t* s16, int8_t* wq, uint16_t* w_scale16);

/* O28: xq = clamp(rne(fl(fl(x * fl(1/dec(s16[j]))) * fl(1/dec(act_scale16)))), +-127). */
void sqo_quant_act_h(const void* x, int xtype, int64_t m, int64_t k,
                     const uint16_t* s16, uint16_t act_scale16, int8_t* xq);

/* O29: y = fl(fl(acc) * fl(dec(act_scale16) * dec(w_scale16[c]))), fp32 or bf16. */
void sqo_dequant_h(const int32_t* acc, int64_t m, int64_t n, uint16_t act_scale16,
                   const uint16_t* w_scale16, int ytype, void* y);

#ifdef __cplusplus
}
#endif
#endif
