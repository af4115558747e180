// sq_kernels.h -- host-side launchers of the libsq kernels. Internal to the
// library: the C ABI in include/sq.h validates arguments and calls these.
// Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sqk {

enum ElemType { kF32 = 0, kBF16 = 1 };

inline int elem_bytes(int t) { return t == kBF16 ? 2 : 4; }

// items per batched call (the projections of one transformer block and more)
constexpr int kMaxBatch = 16;

// column max |x| of x[rows,k] into absmax[k] (overwrite or running max)
hipError_t absmax(const void* x, int xt, int64_t rows, int64_t k, float* absmax, bool accumulate,
                  hipStream_t stream);

// the same for up to kMaxBatch inputs: one zero fill and one reduction launch
struct AbsmaxItem {
    const void* x;
    int xt;
    int64_t rows, k;
    float* absmax;
};
hipError_t absmax_batched(const AbsmaxItem* items, int count, bool accumulate, hipStream_t stream);

// act_scale = fp32(max_j fp32(max(act_max[j], 1e-5) * inv_s[j]) / 127)
hipError_t act_scale(const float* act_max, const float* inv_s, int64_t k, float* act_scale, hipStream_t stream);

// sample_max[b, j] = max over the rows of sample b of |x[., j]| (samples of
// rows_per_sample consecutive rows)
hipError_t sample_max(const void* x, int xt, int64_t samples, int64_t rows_per_sample, int64_t k,
                      float* sample_max, hipStream_t stream);

// sum[j] += sample_max[b, j] in fp64, b ascending
hipError_t sum_samples(const float* sample_max, int64_t samples, int64_t k, double* sum, hipStream_t stream);

// act_max[j] = fp32(sum[j] / count)
hipError_t mean_finalize(const double* sum, int64_t count, int64_t k, float* act_max, hipStream_t stream);

// nearest-rank percentile of |x[:, j]|: the rank-th smallest magnitude (1-based)
size_t percentile_workspace(int xt, int64_t k);
hipError_t percentile(const void* x, int xt, int64_t rows, int64_t k, int64_t rank, void* workspace,
                      float* act_max, hipStream_t stream);
// the same scratch in a static device array of percentile_scratch_bytes()
// (no allocation): its address on the current device
size_t percentile_scratch_bytes();
hipError_t percentile_scratch(void** ptr);

// RMSNorm y = fl(fl(h * r) * gamma) (fp32 or bf16 out), r per row (optional out)
hipError_t rmsnorm(const void* h, int ht, int64_t m, int64_t k, const float* gamma, float eps, void* y, int yt,
                   float* r_out, hipStream_t stream);

// RMSNorm with the folded weight, quantized per tensor in the same pass
hipError_t rmsnorm_quant(const void* h, int ht, int64_t m, int64_t k, const float* gamma_folded, float eps,
                         const float* act_scale, int8_t* xq, float* r_out, hipStream_t stream);
// the same for n <= 4 consumers of one norm output (their own folded weights
// and act scales): one pass over h when the weights fit the registers
hipError_t rmsnorm_quant_multi(const void* h, int ht, int64_t m, int64_t k, float eps, int n,
                               const float* const* gamma_folded, const float* const* act_scale, int8_t* const* xq,
                               float* r_out, hipStream_t stream);

// gamma_folded = fl(gamma * inv_s)
hipError_t fold_norm_weight(const float* gamma, const float* inv_s, int64_t k, float* gamma_folded,
                            hipStream_t stream);

// s, inv_s, act_scale from the two statistics
hipError_t smooth_factors(const float* act_max, const float* w_max, int64_t k, float alpha, float* s,
                          float* inv_s, float* act_scale, hipStream_t stream);

// the same for up to kMaxBatch projections: two launches in all
// h: the fp16 scale storage of ADR-010 "Consequences" (s and act_scale are
// then binary16 arrays, inv_s is not written); otherwise fp32 throughout
struct SmoothItem {
    const float* act_max;
    const float* w_max;
    int64_t k;
    float alpha;
    void* s;
    float* inv_s;
    void* act_scale;
    bool h;
};
hipError_t smooth_factors_batched(const SmoothItem* items, int count, hipStream_t stream);
// the same with the act scale over 448 (e4m3 codes)
hipError_t smooth_factors_fp8_batched(const SmoothItem* items, int count, hipStream_t stream);
// the act scale alone for several items (act_max, inv_s, k, act_scale used)
hipError_t act_scale_batched(const SmoothItem* items, int count, hipStream_t stream);

// W' = W diag(s), per-row symmetric int8 (h: binary16 s and w_scale)
hipError_t quant_weight(const void* w, int wt, int64_t n, int64_t k, const void* s, int8_t* wq,
                        void* w_scale, bool h, hipStream_t stream);

// the same for up to kMaxBatch weights: one persistent launch per kernel
// shape among the items (weights of equal row length share one)
// h: s and w_scale are binary16 (the codes then use the reciprocal of the
// stored row scale, clamped to +-127)
struct QuantWeightItem {
    const void* w;
    int wt;
    int64_t n, k;
    const void* s;
    int8_t* wq;
    void* w_scale;
    bool h;
};
hipError_t quant_weight_batched(const QuantWeightItem* items, int count, hipStream_t stream);

// xq = q8((x * inv_s) * (1/act_scale)) (h: binary16 s in place of inv_s and a
// binary16 act_scale)
hipError_t quant_act(const void* x, int xt, int64_t m, int64_t k, const void* inv_s,
                     const void* act_scale, int8_t* xq, bool h, hipStream_t stream);

// the same for up to kMaxBatch projections in one launch; projections fed by
// the same input read it once
// h: inv_s holds the binary16 s (the kernel forms fl(1 / s) itself) and
// act_scale is binary16
struct ActItem {
    const void* x;
    int xt;
    int64_t m, k;
    const void* inv_s;
    const void* act_scale;
    int8_t* xq;
    bool h;
};
hipError_t quant_act_batched(const ActItem* items, int count, hipStream_t stream);

// y = fp32(acc) * (act_scale * w_scale[n]) in fp32 or bf16, optional int32 acc
// (h: binary16 act_scale and w_scale, decoded before the product)
hipError_t gemm_dequant(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                        const void* act_scale, const void* w_scale, void* y, int yt, int32_t* acc_out, bool h,
                        hipStream_t stream);

// the same for up to kMaxBatch products: those that pick the same large tile
// (and output type) share one launch
struct GemmItem {
    const int8_t* xq;
    const int8_t* wq;
    int64_t m, n, k;
    const void* act_scale;  // fp32, or binary16 when h
    const void* w_scale;    // fp32, or binary16 when h
    void* y;
    int yt;
    void* acc_out;  // int32 for int8 codes, fp32 for e4m3 codes, or NULL
    bool h;
};
hipError_t gemm_dequant_batched(const GemmItem* items, int count, hipStream_t stream);

// FP8 (OCP E4M3) variant: act scale over 448, e4m3 weight and activation
// codes, the e4m3 x e4m3 -> fp32 product with the same dequant epilogue
hipError_t act_scale_fp8(const float* act_max, const float* inv_s, int64_t k, float* act_scale,
                         hipStream_t stream);
hipError_t quant_weight_fp8(const void* w, int wt, int64_t n, int64_t k, const float* s, uint8_t* wq,
                            float* w_scale, hipStream_t stream);
hipError_t quant_act_fp8(const void* x, int xt, int64_t m, int64_t k, const float* inv_s, const float* act_scale,
                         uint8_t* xq, hipStream_t stream);
hipError_t gemm_fp8(const uint8_t* xq, const uint8_t* wq, int64_t m, int64_t n, int64_t k, const float* act_scale,
                    const float* w_scale, void* y, int yt, float* acc_out, hipStream_t stream);
// batched FP8 forms: items as for the int8 forms, with e4m3 code bytes in the
// int8 fields and fp32 accumulators in GemmItem::acc_out
hipError_t quant_weight_fp8_batched(const QuantWeightItem* items, int count, hipStream_t stream);
hipError_t quant_act_fp8_batched(const ActItem* items, int count, hipStream_t stream);
hipError_t gemm_fp8_batched(const GemmItem* items, int count, hipStream_t stream);

// Block tile (rows, columns) the GEMM uses for an m x n output.
void gemm_tiling(int64_t m, int64_t n, int* block_m, int* block_n);
// the tile of each item of a gemm_dequant_batched call (items of one output
// type and scale storage)
void gemm_batched_tiling(const GemmItem* items, int count, int* block_m, int* block_n);

// Number of fp64 partial slots gemm_sse writes for an m x n problem.
int64_t gemm_sse_slots(int64_t m, int64_t n);

// Per-slot partial sums of ((double)y - (double)yref)^2 with y the fp32
// dequantized product; slots[gemm_sse_slots(m,n)] fp64.
hipError_t gemm_sse(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                    const float* act_scale, const float* w_scale, const float* yref, double* slots,
                    hipStream_t stream);

// yref[m,n] = x[m,k] * w[n,k]^T in fp32 (bf16: exact products, fp32 sums)
hipError_t ref_gemm(const void* x, int xt, const void* w, int wt, int64_t m, int64_t n, int64_t k,
                    float* yref, hipStream_t stream);

// the same for nb activation batches x[b] of rows x k against one weight:
// yref + b * rows * n; bf16 batches share one grouped launch (per 16)
hipError_t ref_gemm_batched(const void* const* x, int xt, int nb, int64_t rows, const void* w, int wt, int64_t n,
                            int64_t k, float* yref, hipStream_t stream);

// out[g] = (sum over the slots of group g, in a fixed order) / count, where
// group g is the `per_group` consecutive slots starting at g * per_group
hipError_t reduce_slots(const double* slots, int64_t per_group, int groups, double count, double* out,
                        hipStream_t stream);

}  // namespace sqk
