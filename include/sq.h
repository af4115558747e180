/*
 * sq.h -- C ABI of libsq: the SmoothQuant W8A8 linear-layer path on AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (cited by page and section):
 *   [kwkr]  the Chinese engineering blog on SmoothQuant W8A8 at kwkr.cn
 *           (sections 1.2, 2.1-2.3, 3.1-3.3)
 *   [ADR]   "010. SmoothQuant Integration", blog.yoooo.fun (Context, Decision,
 *           Key design, Consequences)
 *   [pwwt]  "SmoothQuant技术解析：LLM模型INT8无损量化实践", pwwt.cn (§3.1 kernel stub)
 *   [tbr8]  tbr8.org, activation outliers and SmoothQuant (PyTorch example);
 *   [pwwt §2.3] static and dynamic scale modes on the same pwwt.cn page
 *   [aiu]   "SmoothQuant 和激活量化", aiunderstanding.org (the section on where
 *           smoothing goes next: INT8 and FP8 serving)
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major with the reduction dimension k contiguous:
 *     activations X[m,k] (row = token), weights W[n,k] (row = output channel;
 *     column j = input channel j). The layer computes Y[m,n] = sum_j X[m,j]W[n,j].
 *   - Every array pointer is a DEVICE pointer unless marked (host). The caller
 *     owns every buffer; the library allocates nothing and keeps no state
 *     between calls. Device pointers must be 16-byte aligned.
 *   - k must be a positive multiple of 64; m, n, rows may be 0 (then nothing is
 *     launched and SQ_OK is returned; an overwrite of absmax with rows = 0
 *     writes zeros).
 *   - Calls are asynchronous on `stream` (0 = the null stream) unless noted.
 *     Arguments are validated before anything is launched; on any error
 *     nothing is written. A failed launch returns SQ_ERR_HIP.
 *   - fp32 arithmetic is IEEE single precision, round-to-nearest-even, with no
 *     fused multiply-add on the quantization paths. Integer codes are in
 *     [-127, 127]; rounding of codes is half-to-even.
 *   - No exception or abort crosses this interface. Functions are reentrant;
 *     calls on one stream are ordered, calls on different streams that write
 *     the same buffers race.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQ_OK = 0,
    SQ_ERR_NULL = 1,      /* a required pointer is NULL */
    SQ_ERR_SHAPE = 2,     /* negative size, k not a positive multiple of 64, size limit exceeded */
    SQ_ERR_DTYPE = 3,     /* element type not supported for this argument */
    SQ_ERR_ALPHA = 4,     /* alpha not finite or outside [0, 1] */
    SQ_ERR_WORKSPACE = 5, /* workspace missing or smaller than sq_alpha_search_workspace reports */
    SQ_ERR_HIP = 6,       /* a HIP launch or runtime call failed */
    SQ_ERR_ALIGN = 7,     /* a device pointer is not 16-byte aligned */
    SQ_ERR_SCRATCH = 8,   /* the problem needs more than an allocation-free entry point's static scratch */
    /* range sentinels, never returned: any int passed to sq_status_string is a
     * value of the type, in C and in C++ alike */
    SQ_STATUS_RANGE_MIN_ = -2147483647 - 1,
    SQ_STATUS_RANGE_MAX_ = 2147483647
} sq_status;

/* Element types. The two sentinels give the enum the range of a 32-bit int,
 * so any int a caller passes is a value of the type (and is rejected with
 * SQ_ERR_DTYPE unless it is SQ_F32 or SQ_BF16), in C and in C++ alike. */
typedef enum {
    SQ_F32 = 0,
    SQ_BF16 = 1,
    SQ_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    SQ_DTYPE_RANGE_MAX_ = 2147483647
} sq_dtype;

/* Largest k accepted by the GEMM: k*127*127 must stay below 2^31 so the
 * int32 accumulator is exact in any summation order. */
#define SQ_MAX_GEMM_K 131072

/*
 * Per-input-channel max |x| (calibration statistic) [kwkr §3.1; ADR Layer 2,
 * add_batch keeps a running per-channel max-abs]. Also used on the weight
 * W[n,k] (rows = n) to get max|W_j| over output rows.
 *   x       [rows, k] of type xt (SQ_F32 or SQ_BF16)
 *   absmax  [k] fp32, in/out. accumulate = 0: absmax[j] = max_t |x[t,j]|
 *           (0 when rows = 0); accumulate = 1: absmax[j] = max(absmax[j],
 *           max_t |x[t,j]|), the running max over calibration batches.
 * Exact (no rounding). Inputs must be finite.
 */
sq_status sq_calib_absmax(const void* x, sq_dtype xt, int64_t rows, int64_t k,
                          float* absmax, int accumulate, hipStream_t stream);

/*
 * Smoothing factors [kwkr §2.2; ADR Context item 1] and the closed-form
 * per-tensor activation scale [ADR Key design item 1]:
 *   a_j = max(act_max[j], 1e-5), w_j = max(w_max[j], 1e-5)   (floor as in [tbr8])
 *   s[j]      = fp32( a_j^alpha / w_j^(1-alpha) )   (pow and quotient in fp64)
 *   inv_s[j]  = fp32(1 / s[j])                       [kwkr §2.3: multiply by 1/s]
 *   act_scale = fp32( max_j fp32(a_j * inv_s[j]) / 127 )   (one device float)
 *   act_max, w_max  [k] fp32 input; s, inv_s [k] fp32 output; act_scale [1].
 *   alpha must be finite and in [0, 1] (SQ_ERR_ALPHA otherwise) [ADR Key design 3].
 */
sq_status sq_smooth_factors(const float* act_max, const float* w_max, int64_t k,
                            float alpha, float* s, float* inv_s, float* act_scale,
                            hipStream_t stream);

/*
 * Offline weight transform [kwkr §3.2: W' = W diag(s)] and symmetric int8
 * with one scale per output row [ADR Context item 3; kwkr §3.3]:
 *   W'[r,j]    = fp32(W[r,j] * s[j])
 *   w_scale[r] = fp32( max(max_j |W'[r,j]|, 1e-5) / 127 )
 *   wq[r,j]    = clamp(rne(fp32(W'[r,j] * fp32(1/w_scale[r]))), -127, 127)
 *   w [n,k] of type wt; s [k] fp32; wq [n,k] int8 out; w_scale [n] fp32 out.
 */
sq_status sq_quant_weight(const void* w, sq_dtype wt, int64_t n, int64_t k,
                          const float* s, int8_t* wq, float* w_scale,
                          hipStream_t stream);

/*
 * Runtime activation path: scale by 1/s strictly before quantizing
 * [kwkr §3.2, §5.2; ADR Key design items 4-5], symmetric per-tensor int8:
 *   xq[r,j] = clamp(rne(fp32(fp32(x[r,j]*inv_s[j]) * fp32(1/act_scale[0]))), -127, 127)
 *   x [m,k] of type xt; inv_s [k] fp32; act_scale [1] fp32 (device, so the
 *   forward needs no host synchronisation); xq [m,k] int8 out.
 * Values beyond the calibrated range saturate at +-127.
 */
sq_status sq_smooth_quant_act(const void* x, sq_dtype xt, int64_t m, int64_t k,
                              const float* inv_s, const float* act_scale,
                              int8_t* xq, hipStream_t stream);

/*
 * INT8 x INT8 -> INT32 product with the dequantization fused into the
 * epilogue, scales merged before the multiply [pwwt §3.1 kernel stub]:
 *   acc[r,c] = sum_j xq[r,j] * wq[c,j]            (int32, exact)
 *   y[r,c]   = fp32( fp32(acc[r,c]) * fp32(act_scale[0] * w_scale[c]) )
 *   xq [m,k] int8; wq [n,k] int8; act_scale [1]; w_scale [n] fp32;
 *   y [m,n] of type yt (SQ_F32, or SQ_BF16 = round-to-nearest-even of the
 *   fp32 value); acc_out [m,n] int32 or NULL (written when non-NULL).
 *   k <= SQ_MAX_GEMM_K.
 */
sq_status sq_w8a8_gemm(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n,
                       int64_t k, const float* act_scale, const float* w_scale,
                       void* y, sq_dtype yt, int32_t* acc_out, hipStream_t stream);

/*
 * The closed-form per-tensor activation scale alone [ADR Key design item 1],
 * for a statistic gathered after the smoothing factors were fixed (dynamic
 * mode, robust calibration statistics):
 *   act_scale = fp32( max_j fp32(max(act_max[j], 1e-5) * inv_s[j]) / 127 )
 *   act_max, inv_s [k] fp32; act_scale [1] fp32 out (device).
 */
sq_status sq_act_scale(const float* act_max, const float* inv_s, int64_t k,
                       float* act_scale, hipStream_t stream);

/*
 * sq_act_scale for several projections in one launch (host arrays of count
 * <= SQ_MAX_BATCH items; an output may not overlap another item's buffers).
 * With the batched absmax over the live inputs it gives the dynamic mode of a
 * whole block in two launches.
 */
sq_status sq_act_scale_batched(int count, const float* const* act_max, const float* const* inv_s,
                               const int64_t* k, float* const* act_scale, hipStream_t stream);

/*
 * Dynamic mode [pwwt §2.3: scales computed at run time follow the input, at
 * some extra cost per call]: the offline smoothing factors are kept and the
 * per-tensor activation scale is recomputed from the batch being quantized:
 *   live_max[j] = max_t |x[t,j]|                       (0 when m = 0)
 *   act_scale   = sq_act_scale(live_max, inv_s)
 *   xq          = sq_smooth_quant_act(x, inv_s, act_scale)
 *   x [m,k] of type xt; inv_s [k] fp32; live_max [k] fp32 out (the caller's
 *   buffer, left holding the batch statistic); act_scale [1] fp32 out;
 *   xq [m,k] int8 out. x is read twice (statistic, then codes).
 */
sq_status sq_dynamic_quant_act(const void* x, sq_dtype xt, int64_t m, int64_t k,
                               const float* inv_s, float* live_max, float* act_scale,
                               int8_t* xq, hipStream_t stream);

/*
 * Averaged per-sample maxima [kwkr §3.1: averaging the maxima of several
 * samples makes the statistic less sensitive to one extreme sample]:
 *   x holds `samples` consecutive samples of rows_per_sample rows each:
 *   sample_max[b,j] = max over the rows t of sample b of |x[t,j]|
 *                     ([samples, k] fp32 out)
 *   sum[j]         += (double) sample_max[b,j] for b = 0, 1, ... in order
 *                     ([k] fp64 in/out; zero it before the first batch: the
 *                     additions follow the order of the samples across calls)
 * samples may be 0 (nothing happens); rows_per_sample >= 1.
 */
sq_status sq_calib_sample_max_sum(const void* x, sq_dtype xt, int64_t samples,
                                  int64_t rows_per_sample, int64_t k, float* sample_max,
                                  double* sum, hipStream_t stream);

/* act_max[j] = fp32(sum[j] / count), count >= 1 samples seen. */
sq_status sq_calib_mean_finalize(const double* sum, int64_t count, int64_t k,
                                 float* act_max, hipStream_t stream);

/*
 * Percentile statistic [kwkr §3.1: a high percentile such as 99.9% in place of
 * the absolute maximum, trading the clipped extremes for a tighter range],
 * as a nearest rank over the rows:
 *   rank       = min(max(ceil(q * rows), 1), rows)   (q in fp64)
 *   act_max[j] = the rank-th smallest of |x[t,j]| over t   (exact; q = 1 gives the max)
 *   x [rows, k] of type xt, 1 <= rows <= INT32_MAX; q finite in [0, 1]
 *   (SQ_ERR_SHAPE otherwise); workspace: device, at least
 *   sq_calib_percentile_workspace bytes; act_max [k] fp32 out.
 * Reads x twice (bf16) or four times (fp32): one pass per 8-bit digit of the
 * magnitude.
 */
sq_status sq_calib_percentile_workspace(sq_dtype xt, int64_t k, size_t* bytes);
sq_status sq_calib_percentile(const void* x, sq_dtype xt, int64_t rows, int64_t k, double q,
                              void* workspace, size_t workspace_bytes, float* act_max,
                              hipStream_t stream);

/*
 * sq_calib_percentile without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, rules and result as
 * sq_calib_percentile; the scratch (the per-channel digit histograms, prefixes
 * and ranks: sq_calib_percentile_workspace bytes) lives in a static device
 * array of SQ_PERCENTILE_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends. Problems whose scratch exceeds it are rejected with
 * SQ_ERR_SCRATCH before anything is launched (bf16 input: k <= 16320; fp32:
 * k <= 8128). The call allocates nothing and clears the part of the array it
 * uses with a kernel. Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (different streams, or host threads) race.
 */
#define SQ_PERCENTILE_SCRATCH_BYTES (32u << 20)
sq_status sq_calib_percentile_noalloc(const void* x, sq_dtype xt, int64_t rows, int64_t k, double q,
                                      float* act_max, hipStream_t stream);

/*
 * RMSNorm, the norm in front of the projections of a Llama block; its weight
 * is where 1/s can be folded [kwkr §3.2]:
 *   r[t]   = fp32( 1 / sqrt( sum_j h[t,j]^2 / k + eps ) )   (fp64 arithmetic,
 *            one rounding; the additions of the squares are in an unspecified
 *            order, so r can differ from a sequential sum by one fp32 ulp)
 *   y[t,j] = fp32( fp32(h[t,j] * r[t]) * gamma[j] )   (yt SQ_F32 or SQ_BF16 = RNE)
 *   h [m,k] of type ht; gamma [k] fp32; y [m,k]; r_out [m] fp32 or NULL.
 *   eps finite and >= 0 (SQ_ERR_SHAPE otherwise); m <= INT32_MAX.
 */
sq_status sq_rmsnorm(const void* h, sq_dtype ht, int64_t m, int64_t k, const float* gamma,
                     float eps, void* y, sq_dtype yt, float* r_out, hipStream_t stream);

/*
 * 1/s folded into the norm weight, once, offline [kwkr §2.3, §3.2]:
 *   gamma_folded[j] = fp32(gamma[j] * inv_s[j])      ([k] fp32 in and out)
 */
sq_status sq_fold_norm_weight(const float* gamma, const float* inv_s, int64_t k,
                              float* gamma_folded, hipStream_t stream);

/*
 * RMSNorm with the folded weight feeding the per-tensor quantizer in the same
 * pass: the norm's output is already X/s, scaled before it is rounded [kwkr
 * §3.2], so the separate activation pass disappears:
 *   xq[t,j] = clamp(rne(fp32( fp32(fp32(h[t,j]*r[t]) * gamma_folded[j])
 *                             * fp32(1/act_scale[0]) )), -127, 127)
 *   r as in sq_rmsnorm (r_out [m] or NULL); h [m,k] of type ht;
 *   gamma_folded [k] fp32; act_scale [1] fp32; xq [m,k] int8 out.
 */
sq_status sq_rmsnorm_quant_act(const void* h, sq_dtype ht, int64_t m, int64_t k,
                               const float* gamma_folded, float eps, const float* act_scale,
                               int8_t* xq, float* r_out, hipStream_t stream);

/*
 * The same for n <= SQ_MAX_NORM_CONSUMERS consumers of one norm output (q, k
 * and v after the attention norm; gate and up after the MLP norm), each with
 * its own folded weight and act scale: for every consumer c
 *   xq[c][t,j] = clamp(rne(fp32( fp32(fp32(h[t,j]*r[t]) * gamma_folded[c][j])
 *                                * fp32(1/act_scale[c][0]) )), -127, 127)
 * bit-identical to n calls of sq_rmsnorm_quant_act; h is read once when the n
 * folded weights of a row fit in registers, else once per consumer. The
 * arrays are host arrays of n device pointers; r_out [m] or NULL; no output
 * may overlap another buffer of the call (SQ_ERR_SHAPE).
 */
#define SQ_MAX_NORM_CONSUMERS 4
sq_status sq_rmsnorm_quant_act_multi(const void* h, sq_dtype ht, int64_t m, int64_t k, float eps,
                                     int n, const float* const* gamma_folded,
                                     const float* const* act_scale, int8_t* const* xq, float* r_out,
                                     hipStream_t stream);

/*
 * FP8 variant [aiu: smoothing serves FP8 as well as INT8]: the same smoothed
 * path with OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, largest finite 448; round to nearest even; magnitudes past 448 are
 * clamped to 448) in place of int8. Codes are bytes (uint8_t).
 *   sq_act_scale_fp8:        act_scale = fp32( max_j fp32(max(act_max[j],1e-5) * inv_s[j]) / 448 )
 *   sq_quant_weight_fp8:     w_scale[r] = fp32(max(max_j |W'[r,j]|, 1e-5) / 448),
 *                            wq[r,j] = e4m3(fp32(W'[r,j] * fp32(1/w_scale[r]))), W' = W diag(s)
 *   sq_smooth_quant_act_fp8: xq[r,j] = e4m3(fp32(fp32(x[r,j]*inv_s[j]) * fp32(1/act_scale[0])))
 *   sq_fp8_gemm:             acc[r,c] = sum_j e4m3(xq[r,j]) * e4m3(wq[c,j]) on the matrix cores,
 *                            accumulated in fp32; the FP8 instruction aligns each group of
 *                            64 products to the largest and drops low bits, so acc is within
 *                            about 2^-12 of sum_j |products| of the exact sum (not bit-exact);
 *                            y[r,c] = fp32(acc[r,c] * fp32(act_scale[0] * w_scale[c]))
 *                            (yt SQ_F32 or SQ_BF16 = RNE); acc_out [m,n] fp32 or NULL.
 *                            k <= SQ_MAX_GEMM_K.
 * Shapes, alignment and errors as for the int8 entry points.
 */
sq_status sq_act_scale_fp8(const float* act_max, const float* inv_s, int64_t k,
                           float* act_scale, hipStream_t stream);
sq_status sq_quant_weight_fp8(const void* w, sq_dtype wt, int64_t n, int64_t k,
                              const float* s, uint8_t* wq, float* w_scale,
                              hipStream_t stream);
sq_status sq_smooth_quant_act_fp8(const void* x, sq_dtype xt, int64_t m, int64_t k,
                                  const float* inv_s, const float* act_scale,
                                  uint8_t* xq, hipStream_t stream);
sq_status sq_fp8_gemm(const uint8_t* xq, const uint8_t* wq, int64_t m, int64_t n,
                      int64_t k, const float* act_scale, const float* w_scale,
                      void* y, sq_dtype yt, float* acc_out, hipStream_t stream);

/*
 * Batched FP8 forms, for the projections of a block in few launches (the
 * arrays are host arrays of count <= SQ_MAX_BATCH items, validated item by
 * item as the single forms, with the overlap rule of the int8 batched
 * forms): each item is computed exactly as the single call on it.
 *   sq_smooth_factors_fp8_batched:   sq_smooth_factors on each item, with
 *                                    act_scale as sq_act_scale_fp8 (over 448)
 *   sq_quant_weight_fp8_batched:     sq_quant_weight_fp8 on each item
 *   sq_smooth_quant_act_fp8_batched: sq_smooth_quant_act_fp8 on each item
 *                                    (items that share an input read it once)
 *   sq_fp8_gemm_batched:             sq_fp8_gemm on each item (products that
 *                                    pick the same tile share one launch);
 *                                    acc_out NULL or an array of fp32 pointers
 */
sq_status sq_smooth_factors_fp8_batched(int count, const float* const* act_max,
                                        const float* const* w_max, const int64_t* k,
                                        const float* alpha, float* const* s, float* const* inv_s,
                                        float* const* act_scale, hipStream_t stream);
sq_status sq_quant_weight_fp8_batched(int count, const void* const* w, const sq_dtype* wt,
                                      const int64_t* n, const int64_t* k, const float* const* s,
                                      uint8_t* const* wq, float* const* w_scale, hipStream_t stream);
sq_status sq_smooth_quant_act_fp8_batched(int count, const void* const* x, const sq_dtype* xt,
                                          const int64_t* m, const int64_t* k,
                                          const float* const* inv_s, const float* const* act_scale,
                                          uint8_t* const* xq, hipStream_t stream);
sq_status sq_fp8_gemm_batched(int count, const uint8_t* const* xq, const uint8_t* const* wq,
                              const int64_t* m, const int64_t* n, const int64_t* k,
                              const float* const* act_scale, const float* const* w_scale,
                              void* const* y, const sq_dtype* yt, float* const* acc_out,
                              hipStream_t stream);

/*
 * Host-only query: the block tile (rows x columns of Y per workgroup) that
 * sq_w8a8_gemm uses for an m x n output on the current device. The choice
 * depends only on m, n and the device's compute-unit count; it does not change
 * the result (the int32 sums are exact in any order). Launches nothing. For
 * m <= 4 the product runs on the vector ALUs, a workgroup per 4 weight rows:
 * the reported tile is (m rounded up to 1, 2 or 4) x 4; for 4 < m <= 64 the
 * skinny matrix-core kernel: (16, 32 or 64 activation rows) x (16 weight rows,
 * or 48 when m > 32 and n >= 8192).
 */
sq_status sq_gemm_tiling(int64_t m, int64_t n, int* block_m, int* block_n);

/*
 * Host-only query, the batched counterpart of sq_gemm_tiling: the block tile
 * that each product of an sq_w8a8_gemm_batched (or _f16_batched) call with
 * these shapes uses, all items of one output type and scale storage (items
 * that differ in either are grouped apart; query each group on its own).
 * Products that take the pipelined tiles share one width, chosen for the
 * group (on 256 x 256, up to the last three of them may take 256 x 128), so
 * an item's tile here can differ from its sq_gemm_tiling; the others report
 * their sq_gemm_tiling. Launches nothing; the result does not
 * depend on the data (the int32 sums are exact in any order).
 *   count             1 <= count <= SQ_MAX_BATCH (SQ_ERR_SHAPE otherwise)
 *   m, n, k           host arrays of count shapes (m, n >= 0, k > 0)
 *   block_m, block_n  host arrays of count entries, written
 */
sq_status sq_gemm_batched_tiling(int count, const int64_t* m, const int64_t* n, const int64_t* k,
                                 int* block_m, int* block_n);

/*
 * Workspace bytes needed by sq_alpha_search for the given problem (host
 * output *bytes). Pure host computation.
 */
sq_status sq_alpha_search_workspace(int n_batches, int64_t rows_per_batch,
                                    int64_t n, int64_t k, int n_alphas,
                                    size_t* bytes);

/*
 * Per-layer alpha grid search [ADR Key design item 2]: for each alpha in
 * alphas (host array, e.g. {0.25, 0.5, 0.75, 1.0}) run the full layer --
 * act_max over all batches, sq_smooth_factors, sq_quant_weight,
 * sq_smooth_quant_act, sq_w8a8_gemm with fp32 output -- on the kept
 * calibration batches, and score it by the mean squared error against the
 * unquantized product X W^T computed in fp32 (bf16 inputs: exact products,
 * fp32 accumulation):
 *   mse[i] = sum_b sum_r sum_c (y - yref)^2 / (n_batches * rows_per_batch * n)
 *   (squares and sums in fp64); *best = first index attaining the minimum.
 *   x_batches  (host) array of n_batches device pointers, each [rows_per_batch, k] of type xt
 *   w          [n, k] of type wt
 *   workspace  device buffer of at least sq_alpha_search_workspace(...) bytes
 *   mse        (host) [n_alphas] fp64 out; best (host) out.
 * Synchronises `stream` before returning (the results are on the host).
 * 1 <= n_alphas <= 16; every alpha must satisfy the sq_smooth_factors rule.
 */
sq_status sq_alpha_search(const void* const* x_batches, sq_dtype xt, int n_batches,
                          int64_t rows_per_batch, int64_t k, const void* w,
                          sq_dtype wt, int64_t n, const float* alphas, int n_alphas,
                          void* workspace, size_t workspace_bytes, double* mse,
                          int* best, hipStream_t stream);

/*
 * Batched forms, for the several projections of one transformer block
 * (q, k, v, o, gate, up, down): item i of every per-item array describes one
 * call of the single form above (same arguments, same rules), and the results
 * are bit-for-bit those of calling the single form once per item. They exist
 * to cut launches: the items share one pass of each kernel instead of one
 * short launch apiece, so the ramp and drain of a launch are paid once.
 *   count       1 <= count <= SQ_MAX_BATCH (SQ_ERR_SHAPE otherwise)
 *   arrays      every per-item array is a (host) array of count entries;
 *               the pointers in them are device pointers as in the single form
 *   outputs     no item's output range may overlap another item's input or
 *               output range (SQ_ERR_SHAPE); inputs may be shared (q, k and v
 *               read one statistic)
 *   validation  every item is checked as the single form would check it, in
 *               item order, before anything is launched; the first failure is
 *               returned and nothing is written
 *
 * sq_calib_absmax_batched [kwkr §3.1; ADR Layer 2]: absmax[i] = column max of
 *   |x[i]| ([rows[i], k[i]] of type xt[i]); accumulate applies to every item.
 *   One zero fill (overwrite form) and one reduction launch.
 * sq_smooth_factors_batched [kwkr §2.2; ADR Key design items 1, 3]: s[i],
 *   inv_s[i], act_scale[i] from act_max[i], w_max[i] with alpha[i]. Two launches.
 * sq_quant_weight_batched [kwkr §3.2, §3.3; ADR Context item 3]: wq[i],
 *   w_scale[i] from w[i] ([n[i], k[i]] of type wt[i]) and s[i]. One launch per
 *   distinct (element type, row-length class) among the items; the 13B block's
 *   seven weights take two.
 * sq_smooth_quant_act_batched [kwkr §3.2, §5.2; ADR Key design items 4-5]:
 *   xq[i] from x[i] ([m[i], k[i]] of type xt[i]), inv_s[i], act_scale[i]. One
 *   launch; items that name the same input (same pointer, type and shape: q, k
 *   and v, or gate and up) read it once, up to four consumers per pass.
 * sq_w8a8_gemm_batched [pwwt §3.1]: y[i] (type yt[i]) and, when acc_out is
 *   not NULL and acc_out[i] is not NULL, acc_out[i] from xq[i] [m[i], k[i]],
 *   wq[i] [n[i], k[i]], act_scale[i], w_scale[i]. Products that take the
 *   pipelined tiles and share the output type share one launch (the next
 *   product's tiles start as compute units free up) at one tile width, the
 *   one with the least predicted time for the whole group; a launch on
 *   256 x 256 tiles may run up to its last three products on 256 x 128 when
 *   that evens out its last round (sq_gemm_batched_tiling reports each
 *   product's tile); products with m <= 4 (decode: q, k and
 *   v, or gate and up) share one vector-ALU launch when their row class
 *   (m rounded up to 1, 2 or 4), K chunk class and output type match;
 *   products with 4 < m <= 64 share one skinny launch when their skinny
 *   configuration (sq_gemm_tiling) and output type match, unless each alone
 *   already fills the compute units twice over (then a launch each).
 */
#define SQ_MAX_BATCH 16

sq_status sq_calib_absmax_batched(int count, const void* const* x, const sq_dtype* xt,
                                  const int64_t* rows, const int64_t* k, float* const* absmax,
                                  int accumulate, hipStream_t stream);

sq_status sq_smooth_factors_batched(int count, const float* const* act_max,
                                    const float* const* w_max, const int64_t* k,
                                    const float* alpha, float* const* s, float* const* inv_s,
                                    float* const* act_scale, hipStream_t stream);

sq_status sq_quant_weight_batched(int count, const void* const* w, const sq_dtype* wt,
                                  const int64_t* n, const int64_t* k, const float* const* s,
                                  int8_t* const* wq, float* const* w_scale, hipStream_t stream);

sq_status sq_smooth_quant_act_batched(int count, const void* const* x, const sq_dtype* xt,
                                      const int64_t* m, const int64_t* k, const float* const* inv_s,
                                      const float* const* act_scale, int8_t* const* xq,
                                      hipStream_t stream);

sq_status sq_w8a8_gemm_batched(int count, const int8_t* const* xq, const int8_t* const* wq,
                               const int64_t* m, const int64_t* n, const int64_t* k,
                               const float* const* act_scale, const float* const* w_scale,
                               void* const* y, const sq_dtype* yt, int32_t* const* acc_out,
                               hipStream_t stream);

/*
 * fp16 scale storage [ADR "Consequences": per-row weight scale, per-tensor act
 * scale and input_scales kept in fp16; "Decision / Layer 1": input_scales is
 * an fp16 buffer]. The int8 layer with every scale it keeps stored as IEEE
 * binary16 bit patterns (uint16_t arrays): each step is the fp32 entry point
 * fed the DECODED stored values, and every stored scale is
 *   f16(v) = binary16 round-to-nearest-even of fp32 v clamped to [2^-24, 65504]
 * (never zero, never infinite). dec() is the exact decode to fp32.
 *   sq_smooth_factors_f16:   s[j] = f16(s_j), s_j the fp32 factor of
 *                            sq_smooth_factors; no inv_s is stored: its users form
 *                            inv_j = fp32(1 / dec(s[j])) themselves;
 *                            act_scale[0] = f16(fp32(max_j fp32(a_j * inv_j) / 127)).
 *   sq_quant_weight_f16:     W'[r,j] = fp32(W[r,j] * dec(s[j]));
 *                            w_scale[r] = f16(fp32(max(max_j |W'[r,j]|, 1e-5) / 127));
 *                            wq[r,j] = clamp(rne(fp32(W'[r,j] * fp32(1/dec(w_scale[r])))), +-127)
 *                            (the stored scale can sit below the fp32 one, so the
 *                            clamp can act).
 *   sq_smooth_quant_act_f16: xq[r,j] = clamp(rne(fp32(fp32(x[r,j] * inv_j) *
 *                            fp32(1/dec(act_scale[0])))), +-127).
 *   sq_w8a8_gemm_f16:        y[r,c] = fp32(fp32(acc[r,c]) * fp32(dec(act_scale[0]) *
 *                            dec(w_scale[c]))), acc and acc_out as sq_w8a8_gemm.
 * Batched forms: each item exactly as the single call, with the grouping,
 * launch counts and overlap rule of the fp32 batched forms. Shapes, alignment
 * (16 bytes, also for the uint16_t arrays) and errors as for the fp32 entry
 * points; s and act_scale are outputs of sq_smooth_factors_f16 (act_scale one
 * binary16 value in a 16-byte aligned slot).
 */
sq_status sq_smooth_factors_f16(const float* act_max, const float* w_max, int64_t k,
                                float alpha, uint16_t* s, uint16_t* act_scale,
                                hipStream_t stream);
sq_status sq_quant_weight_f16(const void* w, sq_dtype wt, int64_t n, int64_t k,
                              const uint16_t* s, int8_t* wq, uint16_t* w_scale,
                              hipStream_t stream);
sq_status sq_smooth_quant_act_f16(const void* x, sq_dtype xt, int64_t m, int64_t k,
                                  const uint16_t* s, const uint16_t* act_scale,
                                  int8_t* xq, hipStream_t stream);
sq_status sq_w8a8_gemm_f16(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n,
                           int64_t k, const uint16_t* act_scale, const uint16_t* w_scale,
                           void* y, sq_dtype yt, int32_t* acc_out, hipStream_t stream);
sq_status sq_smooth_factors_f16_batched(int count, const float* const* act_max,
                                        const float* const* w_max, const int64_t* k,
                                        const float* alpha, uint16_t* const* s,
                                        uint16_t* const* act_scale, hipStream_t stream);
sq_status sq_quant_weight_f16_batched(int count, const void* const* w, const sq_dtype* wt,
                                      const int64_t* n, const int64_t* k,
                                      const uint16_t* const* s, int8_t* const* wq,
                                      uint16_t* const* w_scale, hipStream_t stream);
sq_status sq_smooth_quant_act_f16_batched(int count, const void* const* x, const sq_dtype* xt,
                                          const int64_t* m, const int64_t* k,
                                          const uint16_t* const* s,
                                          const uint16_t* const* act_scale, int8_t* const* xq,
                                          hipStream_t stream);
sq_status sq_w8a8_gemm_f16_batched(int count, const int8_t* const* xq, const int8_t* const* wq,
                                   const int64_t* m, const int64_t* n, const int64_t* k,
                                   const uint16_t* const* act_scale,
                                   const uint16_t* const* w_scale, void* const* y,
                                   const sq_dtype* yt, int32_t* const* acc_out,
                                   hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* sq_status_string(sq_status status);

#ifdef __cplusplus
}
#endif
#endif /* SQ_H */
