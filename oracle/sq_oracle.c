/*
 * sq_oracle.c -- plain CPU reference for the SmoothQuant W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, by the smoke check and by the
 * CPU-baseline leg of the benchmark; never by the product path. It shares no
 * code with the GPU library. Build: gcc -O2 -ffp-contract=off -fopenmp
 * (see oracle/build.py). Every outer loop parallelised with OpenMP is over
 * independent rows or columns, so results do not depend on the thread count.
 *
 * Step numbering (O1..O11) and citations are in sq_oracle.h.
 */
#include "sq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* The pages' only guard constant: the smoothing factor is clamped to at
 * least 1e-5 (tbr8.org PyTorch example). It is applied to the statistics
 * and to the per-row weight maximum so no scale can be zero. */
#define SQO_FLOOR 1e-5f
#define SQO_QMAX 127.0f

int sqo_num_threads(void) { return omp_get_max_threads(); }

void sqo_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* element i of a float buffer of the given type, widened exactly to fp32 */
static float elem(const void* p, int type, int64_t i) {
    if (type == SQO_BF16) return bf16_bits_to_float(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}

/* symmetric int8 code of an already scaled value (kwkr.cn blog §1.2:
 * x_q = round(x/s)); round half to even, clamp to [-127, 127] */
static int8_t quantize_scaled(float v) {
    float r = rintf(v); /* default rounding mode: nearest, ties to even */
    if (r > SQO_QMAX) r = SQO_QMAX;
    if (r < -SQO_QMAX) r = -SQO_QMAX;
    return (int8_t)r;
}

/* O1 (activations) and O2 (weights): per-input-channel max |.| over rows.
 * kwkr.cn blog §3.1; ADR-010 add_batch keeps a running max per channel. */
void sqo_calib_absmax(const void* x, int xtype, int64_t rows, int64_t k,
                      float* absmax, int accumulate) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < k; ++j) {
        float mx = accumulate ? absmax[j] : 0.0f;
        for (int64_t t = 0; t < rows; ++t) {
            float v = fabsf(elem(x, xtype, t * k + j));
            if (v > mx) mx = v;
        }
        absmax[j] = mx;
    }
}

/* O6: closed-form per-tensor activation scale, ADR-010 "Key design" item 1:
 * max over channels of act_max[j]/s_j, divided by 127. Division by s_j is
 * taken as the product with inv_s[j] (kwkr.cn blog §2.3 allows either). */
float sqo_act_scale(const float* act_max, const float* inv_s, int64_t k) {
    float mx = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        float a = act_max[j] > SQO_FLOOR ? act_max[j] : SQO_FLOOR;
        float v = a * inv_s[j];
        if (v > mx) mx = v;
    }
    return mx / SQO_QMAX;
}

/* O3-O6: s_j = max|X_j|^alpha / max|W_j|^(1-alpha) (kwkr.cn blog §2.2),
 * evaluated in fp64 and rounded once to fp32; inv_s = fl(1/s). */
void sqo_smooth_factors(const float* act_max, const float* w_max, int64_t k,
                        double alpha, float* s, float* inv_s, float* act_scale) {
    for (int64_t j = 0; j < k; ++j) {
        float a = act_max[j] > SQO_FLOOR ? act_max[j] : SQO_FLOOR;
        float w = w_max[j] > SQO_FLOOR ? w_max[j] : SQO_FLOOR;
        double num = pow((double)a, alpha);
        double den = pow((double)w, 1.0 - alpha);
        s[j] = (float)(num / den);
        inv_s[j] = 1.0f / s[j];
    }
    *act_scale = sqo_act_scale(act_max, inv_s, k);
}

/* O7: W' = W*diag(s) offline (kwkr.cn blog §3.2), then symmetric int8 with
 * one scale per output row (ADR-010 "Context" item 3; kwkr.cn blog §3.3). */
void sqo_quant_weight(const void* w, int wtype, int64_t n, int64_t k,
                      const float* s, int8_t* wq, float* w_scale) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        float* row = (float*)malloc((size_t)k * sizeof(float));
        float mx = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            row[j] = elem(w, wtype, r * k + j) * s[j];
            float v = fabsf(row[j]);
            if (v > mx) mx = v;
        }
        if (mx < SQO_FLOOR) mx = SQO_FLOOR;
        float ws = mx / SQO_QMAX;
        float inv_ws = 1.0f / ws;
        for (int64_t j = 0; j < k; ++j) wq[r * k + j] = quantize_scaled(row[j] * inv_ws);
        w_scale[r] = ws;
        free(row);
    }
}

/* O8: runtime x/s (as x*inv_s) strictly before the per-tensor quantizer
 * (kwkr.cn blog §3.2 and §5.2; ADR-010 "Key design" items 4-5). */
void sqo_quant_act(const void* x, int xtype, int64_t m, int64_t k,
                   const float* inv_s, float act_scale, int8_t* xq) {
    float inv_a = 1.0f / act_scale;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        for (int64_t j = 0; j < k; ++j) {
            float smoothed = elem(x, xtype, r * k + j) * inv_s[j];
            xq[r * k + j] = quantize_scaled(smoothed * inv_a);
        }
    }
}

/* O9: the int8 x int8 -> int32 product (pwwt.cn §3.1 kernel signature). */
void sqo_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n,
                  int64_t k, int32_t* acc) {
    int64_t idx;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < m * n; ++idx) {
        int64_t r = idx / n, c = idx % n;
        int64_t sum = 0;
        for (int64_t j = 0; j < k; ++j)
            sum += (int64_t)xq[r * k + j] * (int64_t)wq[c * k + j];
        if (sum > INT32_MAX || sum < INT32_MIN) abort(); /* k too large */
        acc[idx] = (int32_t)sum;
    }
}

/* O10: dequant with the two scales merged first (pwwt.cn §3.1 stub: merge the
 * scale multiplications), then one multiply of the converted accumulator. */
void sqo_dequant(const int32_t* acc, int64_t m, int64_t n, float act_scale,
                 const float* w_scale, int ytype, void* y) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        for (int64_t c = 0; c < n; ++c) {
            float scale = act_scale * w_scale[c];
            float v = (float)acc[r * n + c] * scale;
            if (ytype == SQO_BF16)
                ((uint16_t*)y)[r * n + c] = float_to_bf16_rne(v);
            else
                ((float*)y)[r * n + c] = v;
        }
    }
}

void sqo_ref_gemm(const void* x, int xtype, const void* w, int wtype,
                  int64_t m, int64_t n, int64_t k, float* yref) {
    int64_t idx;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < m * n; ++idx) {
        int64_t r = idx / n, c = idx % n;
        double sum = 0.0;
        for (int64_t j = 0; j < k; ++j)
            sum += (double)elem(x, xtype, r * k + j) * (double)elem(w, wtype, c * k + j);
        yref[idx] = (float)sum;
    }
}

double sqo_sse(const float* y, const float* yref, int64_t m, int64_t n) {
    double* row_sse = (double*)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < n; ++c) {
            double d = (double)y[r * n + c] - (double)yref[r * n + c];
            acc += d * d;
        }
        row_sse[r] = acc;
    }
    double total = 0.0;
    for (r = 0; r < m; ++r) total += row_sse[r];
    free(row_sse);
    return total;
}

/* O11: per-layer alpha grid search with the exact final-layer quantization
 * math (ADR-010 "Key design" item 2). act_max is taken over all batches; the
 * error is the mean squared difference against the reference product on the
 * same batches; ties go to the first alpha in grid order. */
int sqo_alpha_search(const void* const* x_batches, int xtype, int nb,
                     int64_t rows, int64_t k, const void* w, int wtype,
                     int64_t n, const double* alphas, int na, double* mse) {
    float* act_max = (float*)calloc((size_t)k, sizeof(float));
    float* w_max = (float*)calloc((size_t)k, sizeof(float));
    float* s = (float*)malloc((size_t)k * sizeof(float));
    float* inv_s = (float*)malloc((size_t)k * sizeof(float));
    int8_t* wq = (int8_t*)malloc((size_t)(n * k));
    float* w_scale = (float*)malloc((size_t)n * sizeof(float));
    int8_t* xq = (int8_t*)malloc((size_t)(rows * k));
    int32_t* acc = (int32_t*)malloc((size_t)(rows * n) * sizeof(int32_t));
    float* y = (float*)malloc((size_t)(rows * n) * sizeof(float));
    float* yref = (float*)malloc((size_t)(nb * rows * n) * sizeof(float));

    for (int b = 0; b < nb; ++b) sqo_calib_absmax(x_batches[b], xtype, rows, k, act_max, 1);
    sqo_calib_absmax(w, wtype, n, k, w_max, 0);
    for (int b = 0; b < nb; ++b)
        sqo_ref_gemm(x_batches[b], xtype, w, wtype, rows, n, k, yref + (int64_t)b * rows * n);

    int best = 0;
    for (int i = 0; i < na; ++i) {
        float act_scale;
        sqo_smooth_factors(act_max, w_max, k, alphas[i], s, inv_s, &act_scale);
        sqo_quant_weight(w, wtype, n, k, s, wq, w_scale);
        double sse = 0.0;
        for (int b = 0; b < nb; ++b) {
            sqo_quant_act(x_batches[b], xtype, rows, k, inv_s, act_scale, xq);
            sqo_gemm_i32(xq, wq, rows, n, k, acc);
            sqo_dequant(acc, rows, n, act_scale, w_scale, SQO_F32, y);
            sse += sqo_sse(y, yref + (int64_t)b * rows * n, rows, n);
        }
        mse[i] = sse / ((double)nb * (double)rows * (double)n);
        if (mse[i] < mse[best]) best = i;
    }

    free(act_max); free(w_max); free(s); free(inv_s); free(wq); free(w_scale);
    free(xq); free(acc); free(y); free(yref);
    return best;
}

/* O13: dynamic mode (pwwt.cn §2.3): the scale is taken from the batch being
 * quantized instead of the calibration set; the offline s is kept, so the
 * closed form of O6 is applied to this batch's channel maxima. */
void sqo_dynamic_quant_act(const void* x, int xtype, int64_t m, int64_t k,
                           const float* inv_s, int8_t* xq, float* act_scale) {
    float* live = (float*)calloc((size_t)(k > 0 ? k : 1), sizeof(float));
    sqo_calib_absmax(x, xtype, m, k, live, 0);
    float a = sqo_act_scale(live, inv_s, k);
    sqo_quant_act(x, xtype, m, k, inv_s, a, xq);
    *act_scale = a;
    free(live);
}

/* O14: the averaged-maxima statistic of kwkr.cn blog §3.1: the maximum of
 * each calibration sample, averaged over the samples. */
void sqo_calib_sample_max_sum(const void* x, int xtype, int64_t samples,
                              int64_t rows_per_sample, int64_t k, double* sum) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < k; ++j) {
        for (int64_t b = 0; b < samples; ++b) {
            float mx = 0.0f;
            for (int64_t t = 0; t < rows_per_sample; ++t) {
                float v = fabsf(elem(x, xtype, (b * rows_per_sample + t) * k + j));
                if (v > mx) mx = v;
            }
            sum[j] += (double)mx;
        }
    }
}

void sqo_calib_mean_finalize(const double* sum, int64_t count, int64_t k,
                             float* act_max) {
    for (int64_t j = 0; j < k; ++j) act_max[j] = (float)(sum[j] / (double)count);
}

/* O15: the percentile statistic of kwkr.cn blog §3.1 (e.g. 99.9% in place of
 * the absolute maximum), as a nearest rank: the smallest magnitude with at
 * least ceil(q * rows) magnitudes at or below it. */
int64_t sqo_percentile_rank(double q, int64_t rows) {
    int64_t rank = (int64_t)ceil(q * (double)rows);
    if (rank < 1) rank = 1;
    if (rank > rows) rank = rows;
    return rank;
}

static int cmp_float(const void* a, const void* b) {
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

void sqo_calib_percentile(const void* x, int xtype, int64_t rows, int64_t k,
                          double q, float* act_max) {
    int64_t rank = sqo_percentile_rank(q, rows);
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < k; ++j) {
        float* col = (float*)malloc((size_t)rows * sizeof(float));
        for (int64_t t = 0; t < rows; ++t) col[t] = fabsf(elem(x, xtype, t * k + j));
        qsort(col, (size_t)rows, sizeof(float), cmp_float);
        act_max[j] = col[rank - 1];
        free(col);
    }
}

/* O16: RMSNorm, the norm that precedes the projections in a Llama block and
 * whose weight gamma can absorb 1/s (kwkr.cn blog §3.2). */
void sqo_rms_inv(const void* h, int htype, int64_t m, int64_t k, float eps,
                 float* r) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < m; ++t) {
        double ss = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            double v = (double)elem(h, htype, t * k + j);
            ss += v * v;
        }
        r[t] = (float)(1.0 / sqrt(ss / (double)k + (double)eps));
    }
}

void sqo_rmsnorm_apply(const void* h, int htype, int64_t m, int64_t k,
                       const float* r, const float* gamma, int ytype, void* y) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < m; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            float v = (elem(h, htype, t * k + j) * r[t]) * gamma[j];
            if (ytype == SQO_BF16)
                ((uint16_t*)y)[t * k + j] = float_to_bf16_rne(v);
            else
                ((float*)y)[t * k + j] = v;
        }
    }
}

/* O17: kwkr.cn blog §3.2: with a norm in front of the layer, 1/s is
 * multiplied into the norm's gamma once, offline. */
void sqo_fold_norm_weight(const float* gamma, const float* inv_s, int64_t k,
                          float* gamma_folded) {
    for (int64_t j = 0; j < k; ++j) gamma_folded[j] = gamma[j] * inv_s[j];
}

/* O18: the norm output with the folded gamma is already X/s, so it goes
 * straight into the per-tensor quantizer (scaling before quantizing, kwkr.cn
 * blog §3.2). */
void sqo_norm_quant_apply(const void* h, int htype, int64_t m, int64_t k,
                          const float* r, const float* gamma_folded,
                          float act_scale, int8_t* xq) {
    float inv_a = 1.0f / act_scale;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < m; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            float smoothed = (elem(h, htype, t * k + j) * r[t]) * gamma_folded[j];
            xq[t * k + j] = quantize_scaled(smoothed * inv_a);
        }
    }
}

/* O19: OCP FP8 E4M3 -- the 8-bit floating-point target that smoothing also
 * serves (aiunderstanding.org, the section on where SmoothQuant goes next).
 * Normal values (1 + m/8) * 2^(E-7), E = 1..15 (E = 15, m = 7 is NaN);
 * subnormals m * 2^-9. */
uint8_t sqo_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a == 0.0f) return sign;
    int e;
    frexpf(a, &e);               /* a = f * 2^e with f in [0.5, 1) */
    int E = e - 1;               /* a in [2^E, 2^(E+1)) */
    if (E < -6) {                /* below the smallest normal: steps of 2^-9 */
        float q = rintf(ldexpf(a, 9));
        return sign | (uint8_t)q; /* q = 8 is the smallest normal, 0x08 */
    }
    float q = rintf(ldexpf(a, 3 - E)); /* 8 .. 16: the significand in eighths */
    if (q == 16.0f) {
        q = 8.0f;
        E += 1;
    }
    if (E > 8 || (E == 8 && q > 14.0f)) return sign | 0x7e; /* past 448: saturate */
    return sign | (uint8_t)(((E + 7) << 3) | ((int)q - 8));
}

float sqo_e4m3_decode(uint8_t b) {
    int ef = (b >> 3) & 0xf, m = b & 7;
    float mag;
    if ((b & 0x7f) == 0x7f) return NAN;
    if (ef == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, ef - 7);
    return (b & 0x80) ? -mag : mag;
}

#define SQO_FP8_MAX 448.0f

/* O20: O7 with the e4m3 grid in place of the integer one. */
void sqo_quant_weight_fp8(const void* w, int wtype, int64_t n, int64_t k,
                          const float* s, uint8_t* wq, float* w_scale) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        float* row = (float*)malloc((size_t)k * sizeof(float));
        float mx = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            row[j] = s[j] * elem(w, wtype, r * k + j);
            float v = fabsf(row[j]);
            if (v > mx) mx = v;
        }
        mx = mx < SQO_FLOOR ? SQO_FLOOR : mx;
        float ws = mx / SQO_FP8_MAX;
        float inv_ws = 1.0f / ws;
        for (int64_t j = 0; j < k; ++j) wq[r * k + j] = sqo_e4m3_encode(row[j] * inv_ws);
        w_scale[r] = ws;
        free(row);
    }
}

/* O21: O6 with the e4m3 range. */
float sqo_act_scale_fp8(const float* act_max, const float* inv_s, int64_t k) {
    float mx = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        float a = act_max[j] > SQO_FLOOR ? act_max[j] : SQO_FLOOR;
        float v = inv_s[j] * a;
        if (v > mx) mx = v;
    }
    return mx / SQO_FP8_MAX;
}

/* O22: O8 with the e4m3 grid: scale by 1/s first, then by 1/a, then encode. */
void sqo_quant_act_fp8(const void* x, int xtype, int64_t m, int64_t k,
                       const float* inv_s, float act_scale, uint8_t* xq) {
    float inv_a = 1.0f / act_scale;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        for (int64_t j = 0; j < k; ++j) {
            float smoothed = inv_s[j] * elem(x, xtype, r * k + j);
            xq[r * k + j] = sqo_e4m3_encode(smoothed * inv_a);
        }
    }
}

/* O23: the FP8 product: exact fp64 sums of the decoded codes, then the
 * merged-scale dequantization of O10. */
void sqo_gemm_fp8(const uint8_t* xq, const uint8_t* wq, int64_t m, int64_t n,
                  int64_t k, float act_scale, const float* w_scale, int ytype,
                  void* y, double* acc, double* absacc) {
    int64_t idx;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < m * n; ++idx) {
        int64_t r = idx / n, c = idx % n;
        double sum = 0.0, asum = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            double p = (double)sqo_e4m3_decode(xq[r * k + j]) * (double)sqo_e4m3_decode(wq[c * k + j]);
            sum += p;
            asum += fabs(p);
        }
        float scale = w_scale[c] * act_scale;
        float v = (float)sum * scale;
        if (ytype == SQO_BF16)
            ((uint16_t*)y)[idx] = float_to_bf16_rne(v);
        else
            ((float*)y)[idx] = v;
        if (acc) acc[idx] = sum;
        if (absacc) absacc[idx] = asum;
    }
}

/* O24: the dequantization of O10 (pwwt.cn §3.1 stub: merged scales) applied to
 * an fp32 accumulator. */
void sqo_dequant_f32(const float* acc, int64_t m, int64_t n, float act_scale,
                     const float* w_scale, int ytype, void* y) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        for (int64_t c = 0; c < n; ++c) {
            float merged = w_scale[c] * act_scale;
            float v = acc[r * n + c] * merged;
            if (ytype == SQO_BF16)
                ((uint16_t*)y)[r * n + c] = float_to_bf16_rne(v);
            else
                ((float*)y)[r * n + c] = v;
        }
    }
}

/* O25: IEEE binary16 -- the storage precision ADR-010 "Consequences" gives the
 * per-row weight scale, the per-tensor activation scale and the per-channel
 * smoothing factors (input_scales). Normal values (1 + m/1024) * 2^(E-15),
 * E = 1..30; subnormals m * 2^-24; rounding to nearest, ties to even; past
 * the largest finite value (65504) the rounding overflows to infinity. */
uint16_t sqo_f16_encode(float v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    float a = fabsf(v);
    if (isnan(v)) return 0x7e00;
    if (a == 0.0f) return sign;
    if (isinf(a)) return sign | 0x7c00;
    int e;
    frexpf(a, &e);                       /* a = f * 2^e with f in [0.5, 1) */
    int E = e - 1;                       /* a in [2^E, 2^(E+1)) */
    if (E < -14) {                       /* below the smallest normal: steps of 2^-24 */
        float q = rintf(ldexpf(a, 24));  /* exact scaling; rintf rounds half to even */
        return sign | (uint16_t)q;       /* q = 1024 is the smallest normal, 0x0400 */
    }
    float q = rintf(ldexpf(a, 10 - E));  /* 1024 .. 2048: the significand in 1024ths */
    if (q == 2048.0f) {
        q = 1024.0f;
        E += 1;
    }
    if (E > 15) return sign | 0x7c00;    /* overflow: infinity */
    return sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024));
}

float sqo_f16_decode(uint16_t h) {
    int ef = (h >> 10) & 0x1f, m = h & 0x3ff;
    float mag;
    if (ef == 31) mag = m ? NAN : INFINITY;
    else if (ef == 0) mag = ldexpf((float)m, -24);
    else mag = ldexpf(1.0f + (float)m / 1024.0f, ef - 15);
    return (h & 0x8000) ? -mag : mag;
}

/* A scale as stored: positive, kept inside the finite positive range of
 * binary16 ([2^-24, 65504]) so a stored scale is never 0 or infinite, then
 * rounded to nearest even. */
#define SQO_F16_MIN 5.9604644775390625e-08f /* 2^-24 */
#define SQO_F16_MAX 65504.0f
uint16_t sqo_scale_f16(float v) {
    if (v < SQO_F16_MIN) v = SQO_F16_MIN;
    if (v > SQO_F16_MAX) v = SQO_F16_MAX;
    return sqo_f16_encode(v);
}

/* O26: O4 with the smoothing factors stored in fp16 (ADR-010: input_scales
 * is an fp16 buffer, the forward divides by it); the reciprocal every later
 * step uses is that of the stored value, and the closed-form activation scale
 * (O6) is formed from it and then stored in fp16 too. */
void sqo_smooth_factors_h(const float* act_max, const float* w_max, int64_t k,
                          double alpha, uint16_t* s16, uint16_t* act_scale16) {
    float mx = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        float a = act_max[j] > SQO_FLOOR ? act_max[j] : SQO_FLOOR;
        float w = w_max[j] > SQO_FLOOR ? w_max[j] : SQO_FLOOR;
        float s = (float)(pow((double)a, alpha) / pow((double)w, 1.0 - alpha));
        s16[j] = sqo_scale_f16(s);
        float inv = 1.0f / sqo_f16_decode(s16[j]);
        float v = a * inv;
        if (v > mx) mx = v;
    }
    *act_scale16 = sqo_scale_f16(mx / SQO_QMAX);
}

/* O27: O7 with the stored fp16 s folded into W and the row scale stored in
 * fp16; the codes use the reciprocal of the stored row scale. A stored scale
 * may sit below the fp32 one (by up to 2^-11 relative for normal values,
 * more in the subnormal range), so the codes are clamped to +-127. */
void sqo_quant_weight_h(const void* w, int wtype, int64_t n, int64_t k,
                        const uint16_t* s16, int8_t* wq, uint16_t* w_scale16) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        float* row = (float*)malloc((size_t)k * sizeof(float));
        float mx = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            row[j] = elem(w, wtype, r * k + j) * sqo_f16_decode(s16[j]);
            float v = fabsf(row[j]);
            if (v > mx) mx = v;
        }
        w_scale16[r] = sqo_scale_f16((mx < SQO_FLOOR ? SQO_FLOOR : mx) / SQO_QMAX);
        float inv_ws = 1.0f / sqo_f16_decode(w_scale16[r]);
        for (int64_t j = 0; j < k; ++j) wq[r * k + j] = quantize_scaled(row[j] * inv_ws);
        free(row);
    }
}

/* O28: O8 with the stored scales: x times the reciprocal of the stored s_j,
 * then times the reciprocal of the stored activation scale. */
void sqo_quant_act_h(const void* x, int xtype, int64_t m, int64_t k,
                     const uint16_t* s16, uint16_t act_scale16, int8_t* xq) {
    float inv_a = 1.0f / sqo_f16_decode(act_scale16);
    float* inv_s = (float*)malloc((size_t)k * sizeof(float));
    for (int64_t j = 0; j < k; ++j) inv_s[j] = 1.0f / sqo_f16_decode(s16[j]);
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r)
        for (int64_t j = 0; j < k; ++j) xq[r * k + j] = quantize_scaled((elem(x, xtype, r * k + j) * inv_s[j]) * inv_a);
    free(inv_s);
}

/* O29: O10 with the stored scales: c[n] = fl(act_scale * w_scale[n]) from the
 * decoded fp16 values, y = fl(fl(acc) * c[n]). */
void sqo_dequant_h(const int32_t* acc, int64_t m, int64_t n, uint16_t act_scale16,
                   const uint16_t* w_scale16, int ytype, void* y) {
    float a = sqo_f16_decode(act_scale16);
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        for (int64_t c = 0; c < n; ++c) {
            float merged = a * sqo_f16_decode(w_scale16[c]);
            float v = (float)acc[r * n + c] * merged;
            if (ytype == SQO_BF16)
                ((uint16_t*)y)[r * n + c] = float_to_bf16_rne(v);
            else
                ((float*)y)[r * n + c] = v;
        }
    }
}

/* O25 over arrays (the pins feed every binary16 value through it). */
void sqo_f16_encode_array(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = sqo_f16_encode(v[i]);
}

void sqo_f16_decode_array(const uint16_t* h, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = sqo_f16_decode(h[i]);
}
