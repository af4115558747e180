// sq_capi.cpp -- the C ABI of libsq (declared in include/sq.h): argument
// validation, then launches on the caller's stream. No allocation, no state.
#include "sq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "sq_kernels.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_k(int64_t k) { return k > 0 && k % 64 == 0; }

bool valid_dtype(sq_dtype t) { return t == SQ_F32 || t == SQ_BF16; }

bool valid_alpha(float a) { return std::isfinite(a) && a >= 0.0f && a <= 1.0f; }

sq_status hip_status(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

constexpr size_t kAlign = 256;

size_t round_up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

// Workspace layout of the alpha search, in this order, each piece 256-byte aligned.
struct AlphaLayout {
    size_t act_max, w_max, s, inv_s, act_scale, w_scale, mse, slots, wq, xq, yref, total;
};

AlphaLayout alpha_layout(int nb, int64_t rows, int64_t n, int64_t k, int na) {
    AlphaLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += round_up(bytes);
        return at;
    };
    L.act_max = take((size_t)k * 4);
    L.w_max = take((size_t)k * 4);
    L.s = take((size_t)k * 4);
    L.inv_s = take((size_t)k * 4);
    L.act_scale = take(16);
    L.w_scale = take((size_t)n * 4);
    L.mse = take((size_t)na * 8);
    L.slots = take((size_t)na * sqk::gemm_sse_slots((int64_t)nb * rows, n) * 8);
    L.wq = take((size_t)n * k);
    L.xq = take((size_t)nb * rows * k);
    L.yref = take((size_t)nb * rows * n * 4);
    L.total = off;
    return L;
}

sq_status check_absmax(const void* x, sq_dtype xt, int64_t rows, int64_t k, const float* absmax) {
    if (!absmax || (rows > 0 && !x)) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (rows < 0 || !valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(absmax) || (rows > 0 && !aligned16(x))) return SQ_ERR_ALIGN;
    return SQ_OK;
}

// Scale storage of an entry point: fp32 with int8 codes, fp32 with e4m3
// codes, or binary16 with int8 codes (ADR-010 "Consequences").
enum Mode { kI8 = 0, kF8 = 1, kI8H = 2 };

int64_t scale_bytes(Mode md) { return md == kI8H ? 2 : 4; }

// h: binary16 storage, which writes no inv_s (it may be NULL)
sq_status check_smooth(const float* act_max, const float* w_max, int64_t k, float alpha, const void* s,
                       const float* inv_s, const void* act_scale, bool h = false) {
    if (!act_max || !w_max || !s || (!h && !inv_s) || !act_scale) return SQ_ERR_NULL;
    if (!valid_k(k)) return SQ_ERR_SHAPE;
    if (!valid_alpha(alpha)) return SQ_ERR_ALPHA;
    if (!aligned16(act_max) || !aligned16(w_max) || !aligned16(s) || (!h && !aligned16(inv_s)) ||
        !aligned16(act_scale))
        return SQ_ERR_ALIGN;
    return SQ_OK;
}

sq_status check_quant_weight(const void* w, sq_dtype wt, int64_t n, int64_t k, const void* s, const int8_t* wq,
                             const void* w_scale) {
    if (!s || (n > 0 && (!w || !wq || !w_scale))) return SQ_ERR_NULL;
    if (!valid_dtype(wt)) return SQ_ERR_DTYPE;
    if (n < 0 || !valid_k(k) || n > INT32_MAX) return SQ_ERR_SHAPE;
    if (!aligned16(s) || (n > 0 && (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale)))) return SQ_ERR_ALIGN;
    return SQ_OK;
}

sq_status check_quant_act(const void* x, sq_dtype xt, int64_t m, int64_t k, const void* inv_s,
                          const void* act_scale, const int8_t* xq) {
    if (!inv_s || !act_scale || (m > 0 && (!x || !xq))) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (m < 0 || !valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(inv_s) || !aligned16(act_scale) || (m > 0 && (!aligned16(x) || !aligned16(xq))))
        return SQ_ERR_ALIGN;
    return SQ_OK;
}

sq_status check_gemm(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k, const void* act_scale,
                     const void* w_scale, const void* y, sq_dtype yt, const void* acc_out) {
    const bool work = m > 0 && n > 0;
    if (!act_scale || (work && (!xq || !wq || !w_scale || !y))) return SQ_ERR_NULL;
    if (!valid_dtype(yt)) return SQ_ERR_DTYPE;
    if (m < 0 || n < 0 || !valid_k(k) || k > SQ_MAX_GEMM_K) return SQ_ERR_SHAPE;
    // tile counts are int on the device side
    if ((m + 127) / 128 * ((n + 127) / 128) > INT32_MAX / 2) return SQ_ERR_SHAPE;
    if (!aligned16(act_scale) ||
        (work && (!aligned16(xq) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) ||
                  (acc_out && !aligned16(acc_out)))))
        return SQ_ERR_ALIGN;
    return SQ_OK;
}

// Byte ranges named by the items of a batched call: an output range of one
// item may not overlap any range of another item.
struct Ranges {
    struct R {
        int item;
        uintptr_t lo, hi;
        bool out;
    } r[6 * SQ_MAX_BATCH];
    int n = 0;
    void add(int item, const void* p, int64_t bytes, bool out) {
        if (p && bytes > 0) r[n++] = R{item, (uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes, out};
    }
    bool overlap() const {
        for (int a = 0; a < n; ++a)
            for (int b = a + 1; b < n; ++b)
                if (r[a].item != r[b].item && (r[a].out || r[b].out) && r[a].lo < r[b].hi && r[b].lo < r[a].hi)
                    return true;
        return false;
    }
};

}  // namespace

extern "C" {

const char* sq_status_string(sq_status status) {
    switch (status) {
        case SQ_OK: return "ok";
        case SQ_ERR_NULL: return "a required pointer is NULL";
        case SQ_ERR_SHAPE: return "invalid shape (negative size, k not a positive multiple of 64, or a size limit)";
        case SQ_ERR_DTYPE: return "unsupported element type";
        case SQ_ERR_ALPHA: return "alpha must be finite and in [0, 1]";
        case SQ_ERR_WORKSPACE: return "workspace missing or too small";
        case SQ_ERR_HIP: return "HIP launch or runtime error";
        case SQ_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case SQ_ERR_SCRATCH: return "problem larger than the library's static scratch (allocation-free entry point)";
    }
    return "unknown status";
}

sq_status sq_calib_absmax(const void* x, sq_dtype xt, int64_t rows, int64_t k, float* absmax, int accumulate,
                          hipStream_t stream) {
    const sq_status st = check_absmax(x, xt, rows, k, absmax);
    if (st != SQ_OK) return st;
    if (rows == 0 && accumulate) return SQ_OK;
    return hip_status(sqk::absmax(x, xt, rows, k, absmax, accumulate != 0, stream));
}

sq_status sq_smooth_factors(const float* act_max, const float* w_max, int64_t k, float alpha, float* s,
                            float* inv_s, float* act_scale, hipStream_t stream) {
    const sq_status st = check_smooth(act_max, w_max, k, alpha, s, inv_s, act_scale);
    if (st != SQ_OK) return st;
    return hip_status(sqk::smooth_factors(act_max, w_max, k, alpha, s, inv_s, act_scale, stream));
}

sq_status sq_quant_weight(const void* w, sq_dtype wt, int64_t n, int64_t k, const float* s, int8_t* wq,
                          float* w_scale, hipStream_t stream) {
    const sq_status st = check_quant_weight(w, wt, n, k, s, wq, w_scale);
    if (st != SQ_OK) return st;
    return hip_status(sqk::quant_weight(w, wt, n, k, s, wq, w_scale, false, stream));
}

sq_status sq_smooth_factors_f16(const float* act_max, const float* w_max, int64_t k, float alpha, uint16_t* s,
                                uint16_t* act_scale, hipStream_t stream) {
    const sq_status st = check_smooth(act_max, w_max, k, alpha, s, nullptr, act_scale, true);
    if (st != SQ_OK) return st;
    const sqk::SmoothItem item{act_max, w_max, k, alpha, s, nullptr, act_scale, true};
    return hip_status(sqk::smooth_factors_batched(&item, 1, stream));
}

sq_status sq_quant_weight_f16(const void* w, sq_dtype wt, int64_t n, int64_t k, const uint16_t* s, int8_t* wq,
                              uint16_t* w_scale, hipStream_t stream) {
    const sq_status st = check_quant_weight(w, wt, n, k, s, wq, w_scale);
    if (st != SQ_OK) return st;
    return hip_status(sqk::quant_weight(w, wt, n, k, s, wq, w_scale, true, stream));
}

sq_status sq_smooth_quant_act_f16(const void* x, sq_dtype xt, int64_t m, int64_t k, const uint16_t* s,
                                  const uint16_t* act_scale, int8_t* xq, hipStream_t stream) {
    const sq_status st = check_quant_act(x, xt, m, k, s, act_scale, xq);
    if (st != SQ_OK) return st;
    return hip_status(sqk::quant_act(x, xt, m, k, s, act_scale, xq, true, stream));
}

sq_status sq_w8a8_gemm_f16(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                           const uint16_t* act_scale, const uint16_t* w_scale, void* y, sq_dtype yt,
                           int32_t* acc_out, hipStream_t stream) {
    const sq_status st = check_gemm(xq, wq, m, n, k, act_scale, w_scale, y, yt, acc_out);
    if (st != SQ_OK) return st;
    return hip_status(sqk::gemm_dequant(xq, wq, m, n, k, act_scale, w_scale, y, yt, acc_out, true, stream));
}

sq_status sq_calib_absmax_batched(int count, const void* const* x, const sq_dtype* xt, const int64_t* rows,
                                  const int64_t* k, float* const* absmax, int accumulate, hipStream_t stream) {
    if (!x || !xt || !rows || !k || !absmax) return SQ_ERR_NULL;
    if (count < 1 || count > SQ_MAX_BATCH) return SQ_ERR_SHAPE;
    Ranges rg;
    sqk::AbsmaxItem items[SQ_MAX_BATCH];
    int n = 0;
    for (int i = 0; i < count; ++i) {
        const sq_status st = check_absmax(x[i], xt[i], rows[i], k[i], absmax[i]);
        if (st != SQ_OK) return st;
        rg.add(i, absmax[i], k[i] * 4, true);
        rg.add(i, x[i], rows[i] * k[i] * (xt[i] == SQ_BF16 ? 2 : 4), false);
        if (rows[i] == 0 && accumulate) continue;
        items[n++] = sqk::AbsmaxItem{x[i], xt[i], rows[i], k[i], absmax[i]};
    }
    if (rg.overlap()) return SQ_ERR_SHAPE;
    if (n == 0) return SQ_OK;
    return hip_status(sqk::absmax_batched(items, n, accumulate != 0, stream));
}

// s, act_scale: fp32 (kI8, kF8) or binary16 (kI8H) arrays; inv_s is
// ignored (and may be NULL) for kI8H
static sq_status smooth_batched(int count, const float* const* act_max, const float* const* w_max,
                                const int64_t* k, const float* alpha, void* const* s, float* const* inv_s,
                                void* const* act_scale, Mode md, hipStream_t stream) {
    const bool h = md == kI8H;
    if (!act_max || !w_max || !k || !alpha || !s || (!h && !inv_s) || !act_scale) return SQ_ERR_NULL;
    if (count < 1 || count > SQ_MAX_BATCH) return SQ_ERR_SHAPE;
    const int64_t sb = scale_bytes(md);
    Ranges rg;
    sqk::SmoothItem items[SQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        float* is = h ? nullptr : inv_s[i];
        const sq_status st = check_smooth(act_max[i], w_max[i], k[i], alpha[i], s[i], is, act_scale[i], h);
        if (st != SQ_OK) return st;
        rg.add(i, act_max[i], k[i] * 4, false);
        rg.add(i, w_max[i], k[i] * 4, false);
        rg.add(i, s[i], k[i] * sb, true);
        rg.add(i, is, k[i] * 4, true);
        rg.add(i, act_scale[i], sb, true);
        items[i] = sqk::SmoothItem{act_max[i], w_max[i], k[i], alpha[i], s[i], is, act_scale[i], h};
    }
    if (rg.overlap()) return SQ_ERR_SHAPE;
    return hip_status(md == kF8 ? sqk::smooth_factors_fp8_batched(items, count, stream)
                                : sqk::smooth_factors_batched(items, count, stream));
}

sq_status sq_smooth_factors_batched(int count, const float* const* act_max, const float* const* w_max,
                                    const int64_t* k, const float* alpha, float* const* s, float* const* inv_s,
                                    float* const* act_scale, hipStream_t stream) {
    return smooth_batched(count, act_max, w_max, k, alpha, (void* const*)s, inv_s, (void* const*)act_scale, kI8,
                          stream);
}

sq_status sq_smooth_factors_fp8_batched(int count, const float* const* act_max, const float* const* w_max,
                                        const int64_t* k, const float* alpha, float* const* s,
                                        float* const* inv_s, float* const* act_scale, hipStream_t stream) {
    return smooth_batched(count, act_max, w_max, k, alpha, (void* const*)s, inv_s, (void* const*)act_scale, kF8,
                          stream);
}

sq_status sq_smooth_factors_f16_batched(int count, const float* const* act_max, const float* const* w_max,
                                        const int64_t* k, const float* alpha, uint16_t* const* s,
                                        uint16_t* const* act_scale, hipStream_t stream) {
    return smooth_batched(count, act_max, w_max, k, alpha, (void* const*)s, nullptr, (void* const*)act_scale, kI8H,
                          stream);
}

static sq_status quant_weight_batched(int count, const void* const* w, const sq_dtype* wt, const int64_t* n,
                                      const int64_t* k, const void* const* s, int8_t* const* wq,
                                      void* const* w_scale, Mode md, hipStream_t stream) {
    if (!w || !wt || !n || !k || !s || !wq || !w_scale) return SQ_ERR_NULL;
    if (count < 1 || count > SQ_MAX_BATCH) return SQ_ERR_SHAPE;
    const int64_t sb = scale_bytes(md);
    Ranges rg;
    sqk::QuantWeightItem items[SQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        const sq_status st = check_quant_weight(w[i], wt[i], n[i], k[i], s[i], wq[i], w_scale[i]);
        if (st != SQ_OK) return st;
        rg.add(i, w[i], n[i] * k[i] * (wt[i] == SQ_BF16 ? 2 : 4), false);
        rg.add(i, s[i], k[i] * sb, false);
        rg.add(i, wq[i], n[i] * k[i], true);
        rg.add(i, w_scale[i], n[i] * sb, true);
        items[i] = sqk::QuantWeightItem{w[i], wt[i], n[i], k[i], s[i], wq[i], w_scale[i], md == kI8H};
    }
    if (rg.overlap()) return SQ_ERR_SHAPE;
    return hip_status(md == kF8 ? sqk::quant_weight_fp8_batched(items, count, stream)
                                : sqk::quant_weight_batched(items, count, stream));
}

sq_status sq_quant_weight_batched(int count, const void* const* w, const sq_dtype* wt, const int64_t* n,
                                  const int64_t* k, const float* const* s, int8_t* const* wq,
                                  float* const* w_scale, hipStream_t stream) {
    return quant_weight_batched(count, w, wt, n, k, (const void* const*)s, wq, (void* const*)w_scale, kI8, stream);
}

sq_status sq_quant_weight_fp8_batched(int count, const void* const* w, const sq_dtype* wt, const int64_t* n,
                                      const int64_t* k, const float* const* s, uint8_t* const* wq,
                                      float* const* w_scale, hipStream_t stream) {
    return quant_weight_batched(count, w, wt, n, k, (const void* const*)s, (int8_t* const*)wq,
                                (void* const*)w_scale, kF8, stream);
}

sq_status sq_quant_weight_f16_batched(int count, const void* const* w, const sq_dtype* wt, const int64_t* n,
                                      const int64_t* k, const uint16_t* const* s, int8_t* const* wq,
                                      uint16_t* const* w_scale, hipStream_t stream) {
    return quant_weight_batched(count, w, wt, n, k, (const void* const*)s, wq, (void* const*)w_scale, kI8H, stream);
}

sq_status sq_smooth_quant_act(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* inv_s,
                              const float* act_scale, int8_t* xq, hipStream_t stream) {
    const sq_status st = check_quant_act(x, xt, m, k, inv_s, act_scale, xq);
    if (st != SQ_OK) return st;
    return hip_status(sqk::quant_act(x, xt, m, k, inv_s, act_scale, xq, false, stream));
}

// inv_s: fp32 inv_s (kI8, kF8) or the binary16 s itself (kI8H)
static sq_status quant_act_batched(int count, const void* const* x, const sq_dtype* xt, const int64_t* m,
                                   const int64_t* k, const void* const* inv_s, const void* const* act_scale,
                                   int8_t* const* xq, Mode md, hipStream_t stream) {
    if (!x || !xt || !m || !k || !inv_s || !act_scale || !xq) return SQ_ERR_NULL;
    if (count < 1 || count > SQ_MAX_BATCH) return SQ_ERR_SHAPE;
    const int64_t sb = scale_bytes(md);
    Ranges rg;
    sqk::ActItem items[SQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        const sq_status st = check_quant_act(x[i], xt[i], m[i], k[i], inv_s[i], act_scale[i], xq[i]);
        if (st != SQ_OK) return st;
        rg.add(i, x[i], m[i] * k[i] * (xt[i] == SQ_BF16 ? 2 : 4), false);
        rg.add(i, inv_s[i], k[i] * sb, false);
        rg.add(i, act_scale[i], sb, false);
        rg.add(i, xq[i], m[i] * k[i], true);
        items[i] = sqk::ActItem{x[i], xt[i], m[i], k[i], inv_s[i], act_scale[i], xq[i], md == kI8H};
    }
    if (rg.overlap()) return SQ_ERR_SHAPE;
    return hip_status(md == kF8 ? sqk::quant_act_fp8_batched(items, count, stream)
                                : sqk::quant_act_batched(items, count, stream));
}

sq_status sq_smooth_quant_act_batched(int count, const void* const* x, const sq_dtype* xt, const int64_t* m,
                                      const int64_t* k, const float* const* inv_s, const float* const* act_scale,
                                      int8_t* const* xq, hipStream_t stream) {
    return quant_act_batched(count, x, xt, m, k, (const void* const*)inv_s, (const void* const*)act_scale, xq, kI8,
                             stream);
}

sq_status sq_smooth_quant_act_fp8_batched(int count, const void* const* x, const sq_dtype* xt, const int64_t* m,
                                          const int64_t* k, const float* const* inv_s,
                                          const float* const* act_scale, uint8_t* const* xq, hipStream_t stream) {
    return quant_act_batched(count, x, xt, m, k, (const void* const*)inv_s, (const void* const*)act_scale,
                             (int8_t* const*)xq, kF8, stream);
}

sq_status sq_smooth_quant_act_f16_batched(int count, const void* const* x, const sq_dtype* xt, const int64_t* m,
                                          const int64_t* k, const uint16_t* const* s,
                                          const uint16_t* const* act_scale, int8_t* const* xq, hipStream_t stream) {
    return quant_act_batched(count, x, xt, m, k, (const void* const*)s, (const void* const*)act_scale, xq, kI8H,
                             stream);
}

sq_status sq_w8a8_gemm(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                       const float* act_scale, const float* w_scale, void* y, sq_dtype yt, int32_t* acc_out,
                       hipStream_t stream) {
    const sq_status st = check_gemm(xq, wq, m, n, k, act_scale, w_scale, y, yt, acc_out);
    if (st != SQ_OK) return st;
    return hip_status(sqk::gemm_dequant(xq, wq, m, n, k, act_scale, w_scale, y, yt, acc_out, false, stream));
}

// acc_out: int32 (int8 codes) or fp32 (e4m3 codes) accumulators, 4 bytes each;
// act_scale, w_scale: fp32, or binary16 (kI8H)
static sq_status gemm_batched(int count, const int8_t* const* xq, const int8_t* const* wq, const int64_t* m,
                              const int64_t* n, const int64_t* k, const void* const* act_scale,
                              const void* const* w_scale, void* const* y, const sq_dtype* yt,
                              void* const* acc_out, Mode md, hipStream_t stream) {
    if (!xq || !wq || !m || !n || !k || !act_scale || !w_scale || !y || !yt) return SQ_ERR_NULL;
    if (count < 1 || count > SQ_MAX_BATCH) return SQ_ERR_SHAPE;
    const int64_t sb = scale_bytes(md);
    Ranges rg;
    sqk::GemmItem items[SQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        void* acc = acc_out ? acc_out[i] : nullptr;
        const sq_status st = check_gemm(xq[i], wq[i], m[i], n[i], k[i], act_scale[i], w_scale[i], y[i], yt[i], acc);
        if (st != SQ_OK) return st;
        rg.add(i, xq[i], m[i] * k[i], false);
        rg.add(i, wq[i], n[i] * k[i], false);
        rg.add(i, act_scale[i], sb, false);
        rg.add(i, w_scale[i], n[i] * sb, false);
        rg.add(i, y[i], m[i] * n[i] * (yt[i] == SQ_BF16 ? 2 : 4), true);
        rg.add(i, acc, m[i] * n[i] * 4, true);
        items[i] =
            sqk::GemmItem{xq[i], wq[i], m[i], n[i], k[i], act_scale[i], w_scale[i], y[i], yt[i], acc, md == kI8H};
    }
    if (rg.overlap()) return SQ_ERR_SHAPE;
    return hip_status(md == kF8 ? sqk::gemm_fp8_batched(items, count, stream)
                                : sqk::gemm_dequant_batched(items, count, stream));
}

sq_status sq_w8a8_gemm_batched(int count, const int8_t* const* xq, const int8_t* const* wq, const int64_t* m,
                               const int64_t* n, const int64_t* k, const float* const* act_scale,
                               const float* const* w_scale, void* const* y, const sq_dtype* yt,
                               int32_t* const* acc_out, hipStream_t stream) {
    return gemm_batched(count, xq, wq, m, n, k, (const void* const*)act_scale, (const void* const*)w_scale, y, yt,
                        (void* const*)acc_out, kI8, stream);
}

sq_status sq_fp8_gemm_batched(int count, const uint8_t* const* xq, const uint8_t* const* wq, const int64_t* m,
                              const int64_t* n, const int64_t* k, const float* const* act_scale,
                              const float* const* w_scale, void* const* y, const sq_dtype* yt,
                              float* const* acc_out, hipStream_t stream) {
    return gemm_batched(count, (const int8_t* const*)xq, (const int8_t* const*)wq, m, n, k,
                        (const void* const*)act_scale, (const void* const*)w_scale, y, yt, (void* const*)acc_out, kF8,
                        stream);
}

sq_status sq_w8a8_gemm_f16_batched(int count, const int8_t* const* xq, const int8_t* const* wq, const int64_t* m,
                                   const int64_t* n, const int64_t* k, const uint16_t* const* act_scale,
                                   const uint16_t* const* w_scale, void* const* y, const sq_dtype* yt,
                                   int32_t* const* acc_out, hipStream_t stream) {
    return gemm_batched(count, xq, wq, m, n, k, (const void* const*)act_scale, (const void* const*)w_scale, y, yt,
                        (void* const*)acc_out, kI8H, stream);
}

sq_status sq_act_scale(const float* act_max, const float* inv_s, int64_t k, float* act_scale, hipStream_t stream) {
    if (!act_max || !inv_s || !act_scale) return SQ_ERR_NULL;
    if (!valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(act_max) || !aligned16(inv_s) || !aligned16(act_scale)) return SQ_ERR_ALIGN;
    return hip_status(sqk::act_scale(act_max, inv_s, k, act_scale, stream));
}

sq_status sq_act_scale_batched(int count, const float* const* act_max, const float* const* inv_s, const int64_t* k,
                               float* const* act_scale, hipStream_t stream) {
    if (!act_max || !inv_s || !k || !act_scale) return SQ_ERR_NULL;
    if (count < 1 || count > SQ_MAX_BATCH) return SQ_ERR_SHAPE;
    Ranges rg;
    sqk::SmoothItem items[SQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        if (!act_max[i] || !inv_s[i] || !act_scale[i]) return SQ_ERR_NULL;
        if (!valid_k(k[i])) return SQ_ERR_SHAPE;
        if (!aligned16(act_max[i]) || !aligned16(inv_s[i]) || !aligned16(act_scale[i])) return SQ_ERR_ALIGN;
        rg.add(i, act_max[i], k[i] * 4, false);
        rg.add(i, inv_s[i], k[i] * 4, false);
        rg.add(i, act_scale[i], 4, true);
        // act_scale_batched only reads inv_s (the field is an output of the smoothing kernels)
        items[i] = sqk::SmoothItem{act_max[i], nullptr, k[i], 0.0f, nullptr, const_cast<float*>(inv_s[i]),
                                   act_scale[i], false};
    }
    if (rg.overlap()) return SQ_ERR_SHAPE;
    return hip_status(sqk::act_scale_batched(items, count, stream));
}

sq_status sq_dynamic_quant_act(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* inv_s,
                               float* live_max, float* act_scale, int8_t* xq, hipStream_t stream) {
    if (!inv_s || !live_max || !act_scale || (m > 0 && (!x || !xq))) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (m < 0 || !valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(inv_s) || !aligned16(live_max) || !aligned16(act_scale) ||
        (m > 0 && (!aligned16(x) || !aligned16(xq))))
        return SQ_ERR_ALIGN;
    hipError_t e = sqk::absmax(x, xt, m, k, live_max, false, stream);
    if (e == hipSuccess) e = sqk::act_scale(live_max, inv_s, k, act_scale, stream);
    if (e == hipSuccess && m > 0) e = sqk::quant_act(x, xt, m, k, inv_s, act_scale, xq, false, stream);
    return hip_status(e);
}

sq_status sq_calib_sample_max_sum(const void* x, sq_dtype xt, int64_t samples, int64_t rows_per_sample, int64_t k,
                                  float* sample_max, double* sum, hipStream_t stream) {
    if (!sum || (samples > 0 && (!x || !sample_max))) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (samples < 0 || rows_per_sample < 1 || !valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(sum) || (samples > 0 && (!aligned16(x) || !aligned16(sample_max)))) return SQ_ERR_ALIGN;
    if (samples == 0) return SQ_OK;
    hipError_t e = sqk::sample_max(x, xt, samples, rows_per_sample, k, sample_max, stream);
    if (e == hipSuccess) e = sqk::sum_samples(sample_max, samples, k, sum, stream);
    return hip_status(e);
}

sq_status sq_calib_mean_finalize(const double* sum, int64_t count, int64_t k, float* act_max, hipStream_t stream) {
    if (!sum || !act_max) return SQ_ERR_NULL;
    if (count < 1 || !valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(sum) || !aligned16(act_max)) return SQ_ERR_ALIGN;
    return hip_status(sqk::mean_finalize(sum, count, k, act_max, stream));
}

sq_status sq_act_scale_fp8(const float* act_max, const float* inv_s, int64_t k, float* act_scale,
                           hipStream_t stream) {
    if (!act_max || !inv_s || !act_scale) return SQ_ERR_NULL;
    if (!valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(act_max) || !aligned16(inv_s) || !aligned16(act_scale)) return SQ_ERR_ALIGN;
    return hip_status(sqk::act_scale_fp8(act_max, inv_s, k, act_scale, stream));
}

sq_status sq_quant_weight_fp8(const void* w, sq_dtype wt, int64_t n, int64_t k, const float* s, uint8_t* wq,
                              float* w_scale, hipStream_t stream) {
    if (!s || (n > 0 && (!w || !wq || !w_scale))) return SQ_ERR_NULL;
    if (!valid_dtype(wt)) return SQ_ERR_DTYPE;
    if (n < 0 || !valid_k(k) || n > INT32_MAX) return SQ_ERR_SHAPE;
    if (!aligned16(s) || (n > 0 && (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale)))) return SQ_ERR_ALIGN;
    return hip_status(sqk::quant_weight_fp8(w, wt, n, k, s, wq, w_scale, stream));
}

sq_status sq_smooth_quant_act_fp8(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* inv_s,
                                  const float* act_scale, uint8_t* xq, hipStream_t stream) {
    if (!inv_s || !act_scale || (m > 0 && (!x || !xq))) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (m < 0 || !valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(inv_s) || !aligned16(act_scale) || (m > 0 && (!aligned16(x) || !aligned16(xq))))
        return SQ_ERR_ALIGN;
    if (m == 0) return SQ_OK;
    return hip_status(sqk::quant_act_fp8(x, xt, m, k, inv_s, act_scale, xq, stream));
}

sq_status sq_fp8_gemm(const uint8_t* xq, const uint8_t* wq, int64_t m, int64_t n, int64_t k, const float* act_scale,
                      const float* w_scale, void* y, sq_dtype yt, float* acc_out, hipStream_t stream) {
    const bool work = m > 0 && n > 0;
    if (!act_scale || (work && (!xq || !wq || !w_scale || !y))) return SQ_ERR_NULL;
    if (!valid_dtype(yt)) return SQ_ERR_DTYPE;
    if (m < 0 || n < 0 || !valid_k(k) || k > SQ_MAX_GEMM_K) return SQ_ERR_SHAPE;
    if ((m + 127) / 128 * ((n + 127) / 128) > INT32_MAX / 2) return SQ_ERR_SHAPE;
    if (!aligned16(act_scale) ||
        (work && (!aligned16(xq) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) ||
                  (acc_out && !aligned16(acc_out)))))
        return SQ_ERR_ALIGN;
    return hip_status(sqk::gemm_fp8(xq, wq, m, n, k, act_scale, w_scale, y, yt, acc_out, stream));
}

sq_status sq_calib_percentile_workspace(sq_dtype xt, int64_t k, size_t* bytes) {
    if (!bytes) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (!valid_k(k)) return SQ_ERR_SHAPE;
    *bytes = sqk::percentile_workspace(xt, k);
    return SQ_OK;
}

sq_status sq_calib_percentile(const void* x, sq_dtype xt, int64_t rows, int64_t k, double q, void* workspace,
                              size_t workspace_bytes, float* act_max, hipStream_t stream) {
    if (!x || !act_max) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (rows < 1 || rows > INT32_MAX || !valid_k(k) || !std::isfinite(q) || q < 0.0 || q > 1.0) return SQ_ERR_SHAPE;
    if (!workspace || workspace_bytes < sqk::percentile_workspace(xt, k)) return SQ_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(act_max) || !aligned16(workspace)) return SQ_ERR_ALIGN;
    int64_t rank = (int64_t)std::ceil(q * (double)rows);
    rank = rank < 1 ? 1 : (rank > rows ? rows : rank);
    return hip_status(sqk::percentile(x, xt, rows, k, rank, workspace, act_max, stream));
}

sq_status sq_calib_percentile_noalloc(const void* x, sq_dtype xt, int64_t rows, int64_t k, double q,
                                      float* act_max, hipStream_t stream) {
    if (!x || !act_max) return SQ_ERR_NULL;
    if (!valid_dtype(xt)) return SQ_ERR_DTYPE;
    if (rows < 1 || rows > INT32_MAX || !valid_k(k) || !std::isfinite(q) || q < 0.0 || q > 1.0) return SQ_ERR_SHAPE;
    if (sqk::percentile_workspace(xt, k) > sqk::percentile_scratch_bytes()) return SQ_ERR_SCRATCH;
    if (!aligned16(x) || !aligned16(act_max)) return SQ_ERR_ALIGN;
    void* scratch = nullptr;
    if (sqk::percentile_scratch(&scratch) != hipSuccess) return SQ_ERR_HIP;
    int64_t rank = (int64_t)std::ceil(q * (double)rows);
    rank = rank < 1 ? 1 : (rank > rows ? rows : rank);
    return hip_status(sqk::percentile(x, xt, rows, k, rank, scratch, act_max, stream));
}

static bool valid_eps(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

sq_status sq_rmsnorm(const void* h, sq_dtype ht, int64_t m, int64_t k, const float* gamma, float eps, void* y,
                     sq_dtype yt, float* r_out, hipStream_t stream) {
    if (!gamma || (m > 0 && (!h || !y))) return SQ_ERR_NULL;
    if (!valid_dtype(ht) || !valid_dtype(yt)) return SQ_ERR_DTYPE;
    if (m < 0 || m > INT32_MAX || !valid_k(k) || !valid_eps(eps)) return SQ_ERR_SHAPE;
    if (!aligned16(gamma) || (m > 0 && (!aligned16(h) || !aligned16(y))) || (r_out && !aligned16(r_out)))
        return SQ_ERR_ALIGN;
    return hip_status(sqk::rmsnorm(h, ht, m, k, gamma, eps, y, yt, r_out, stream));
}

sq_status sq_fold_norm_weight(const float* gamma, const float* inv_s, int64_t k, float* gamma_folded,
                              hipStream_t stream) {
    if (!gamma || !inv_s || !gamma_folded) return SQ_ERR_NULL;
    if (!valid_k(k)) return SQ_ERR_SHAPE;
    if (!aligned16(gamma) || !aligned16(inv_s) || !aligned16(gamma_folded)) return SQ_ERR_ALIGN;
    return hip_status(sqk::fold_norm_weight(gamma, inv_s, k, gamma_folded, stream));
}

sq_status sq_rmsnorm_quant_act(const void* h, sq_dtype ht, int64_t m, int64_t k, const float* gamma_folded,
                               float eps, const float* act_scale, int8_t* xq, float* r_out, hipStream_t stream) {
    if (!gamma_folded || !act_scale || (m > 0 && (!h || !xq))) return SQ_ERR_NULL;
    if (!valid_dtype(ht)) return SQ_ERR_DTYPE;
    if (m < 0 || m > INT32_MAX || !valid_k(k) || !valid_eps(eps)) return SQ_ERR_SHAPE;
    if (!aligned16(gamma_folded) || !aligned16(act_scale) || (m > 0 && (!aligned16(h) || !aligned16(xq))) ||
        (r_out && !aligned16(r_out)))
        return SQ_ERR_ALIGN;
    return hip_status(sqk::rmsnorm_quant(h, ht, m, k, gamma_folded, eps, act_scale, xq, r_out, stream));
}

sq_status sq_rmsnorm_quant_act_multi(const void* h, sq_dtype ht, int64_t m, int64_t k, float eps, int n,
                                     const float* const* gamma_folded, const float* const* act_scale,
                                     int8_t* const* xq, float* r_out, hipStream_t stream) {
    if (!gamma_folded || !act_scale || !xq || (m > 0 && !h)) return SQ_ERR_NULL;
    if (!valid_dtype(ht)) return SQ_ERR_DTYPE;
    if (n < 1 || n > SQ_MAX_NORM_CONSUMERS || m < 0 || m > INT32_MAX || !valid_k(k) || !valid_eps(eps))
        return SQ_ERR_SHAPE;
    if (m > 0 && !aligned16(h)) return SQ_ERR_ALIGN;
    if (r_out && !aligned16(r_out)) return SQ_ERR_ALIGN;
    Ranges rg;  // every buffer its own id: an output may overlap no other buffer
    rg.add(0, h, m * k * (ht == SQ_BF16 ? 2 : 4), false);
    rg.add(1, r_out, m * 4, true);
    for (int c = 0; c < n; ++c) {
        if (!gamma_folded[c] || !act_scale[c] || (m > 0 && !xq[c])) return SQ_ERR_NULL;
        if (!aligned16(gamma_folded[c]) || !aligned16(act_scale[c]) || (m > 0 && !aligned16(xq[c])))
            return SQ_ERR_ALIGN;
        rg.add(2 + 3 * c, gamma_folded[c], k * 4, false);
        rg.add(3 + 3 * c, act_scale[c], 4, false);
        rg.add(4 + 3 * c, xq[c], m * k, true);
    }
    if (rg.overlap()) return SQ_ERR_SHAPE;
    return hip_status(sqk::rmsnorm_quant_multi(h, ht, m, k, eps, n, gamma_folded, act_scale, xq, r_out, stream));
}

sq_status sq_gemm_tiling(int64_t m, int64_t n, int* block_m, int* block_n) {
    if (!block_m || !block_n) return SQ_ERR_NULL;
    if (m < 0 || n < 0) return SQ_ERR_SHAPE;
    sqk::gemm_tiling(m, n, block_m, block_n);
    return SQ_OK;
}

sq_status sq_gemm_batched_tiling(int count, const int64_t* m, const int64_t* n, const int64_t* k, int* block_m,
                                 int* block_n) {
    if (!m || !n || !k || !block_m || !block_n) return SQ_ERR_NULL;
    if (count < 1 || count > SQ_MAX_BATCH) return SQ_ERR_SHAPE;
    sqk::GemmItem items[SQ_MAX_BATCH] = {};
    for (int i = 0; i < count; ++i) {
        if (m[i] < 0 || n[i] < 0 || k[i] < 1) return SQ_ERR_SHAPE;
        items[i].m = m[i];
        items[i].n = n[i];
        items[i].k = k[i];
    }
    sqk::gemm_batched_tiling(items, count, block_m, block_n);
    return SQ_OK;
}

sq_status sq_alpha_search_workspace(int n_batches, int64_t rows_per_batch, int64_t n, int64_t k, int n_alphas,
                                    size_t* bytes) {
    if (!bytes) return SQ_ERR_NULL;
    if (n_batches < 1 || rows_per_batch < 1 || n < 1 || !valid_k(k) || k > SQ_MAX_GEMM_K) return SQ_ERR_SHAPE;
    if (n_alphas < 1 || n_alphas > 16) return SQ_ERR_SHAPE;
    *bytes = alpha_layout(n_batches, rows_per_batch, n, k, n_alphas).total;
    return SQ_OK;
}

sq_status sq_alpha_search(const void* const* x_batches, sq_dtype xt, int n_batches, int64_t rows_per_batch,
                          int64_t k, const void* w, sq_dtype wt, int64_t n, const float* alphas, int n_alphas,
                          void* workspace, size_t workspace_bytes, double* mse, int* best, hipStream_t stream) {
    if (!x_batches || !w || !alphas || !mse || !best) return SQ_ERR_NULL;
    if (!valid_dtype(xt) || !valid_dtype(wt) || xt != wt) return SQ_ERR_DTYPE;
    size_t need = 0;
    sq_status st = sq_alpha_search_workspace(n_batches, rows_per_batch, n, k, n_alphas, &need);
    if (st != SQ_OK) return st;
    if (n > INT32_MAX) return SQ_ERR_SHAPE;
    for (int b = 0; b < n_batches; ++b) {
        if (!x_batches[b]) return SQ_ERR_NULL;
        if (!aligned16(x_batches[b])) return SQ_ERR_ALIGN;
    }
    for (int i = 0; i < n_alphas; ++i)
        if (!valid_alpha(alphas[i])) return SQ_ERR_ALPHA;
    if (!workspace || workspace_bytes < need) return SQ_ERR_WORKSPACE;
    if (!aligned16(w) || !aligned16(workspace)) return SQ_ERR_ALIGN;

    const AlphaLayout L = alpha_layout(n_batches, rows_per_batch, n, k, n_alphas);
    char* base = (char*)workspace;
    float* act_max = (float*)(base + L.act_max);
    float* w_max = (float*)(base + L.w_max);
    float* s = (float*)(base + L.s);
    float* inv_s = (float*)(base + L.inv_s);
    float* act_scale = (float*)(base + L.act_scale);
    float* w_scale = (float*)(base + L.w_scale);
    double* mse_dev = (double*)(base + L.mse);
    double* slots = (double*)(base + L.slots);
    int8_t* wq = (int8_t*)(base + L.wq);
    int8_t* xq = (int8_t*)(base + L.xq);
    float* yref = (float*)(base + L.yref);
    const int64_t rows_total = (int64_t)n_batches * rows_per_batch;
    const int64_t per_gemm = sqk::gemm_sse_slots(rows_total, n);

    hipError_t e = hipSuccess;
    auto run = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
    };
    // statistics over all kept batches, then the reference products
    for (int b = 0; b < n_batches; ++b)
        run(sqk::absmax(x_batches[b], xt, rows_per_batch, k, act_max, b > 0, stream));
    run(sqk::absmax(w, wt, n, k, w_max, false, stream));
    run(sqk::ref_gemm_batched(x_batches, xt, n_batches, rows_per_batch, w, wt, n, k, yref, stream));
    // One full quantized forward per alpha, scored in the GEMM epilogue. The
    // batches' codes are stacked (batch b at rows b * rows_per_batch, as the
    // reference products are), so one product covers every batch.
    for (int i = 0; i < n_alphas && e == hipSuccess; ++i) {
        run(sqk::smooth_factors(act_max, w_max, k, alphas[i], s, inv_s, act_scale, stream));
        run(sqk::quant_weight(w, wt, n, k, s, wq, w_scale, false, stream));
        for (int b0 = 0; b0 < n_batches; b0 += sqk::kMaxBatch) {
            sqk::ActItem items[sqk::kMaxBatch];
            int cnt = 0;
            for (int b = b0; b < n_batches && b < b0 + sqk::kMaxBatch; ++b)
                items[cnt++] = sqk::ActItem{x_batches[b], xt, rows_per_batch, k, inv_s, act_scale,
                                            xq + (int64_t)b * rows_per_batch * k, false};
            run(sqk::quant_act_batched(items, cnt, stream));
        }
        run(sqk::gemm_sse(xq, wq, rows_total, n, k, act_scale, w_scale, yref, slots + (int64_t)i * per_gemm,
                          stream));
    }
    const double count = (double)rows_total * (double)n;
    run(sqk::reduce_slots(slots, per_gemm, n_alphas, count, mse_dev, stream));
    if (e != hipSuccess) return SQ_ERR_HIP;
    run(hipMemcpyAsync(mse, mse_dev, (size_t)n_alphas * sizeof(double), hipMemcpyDeviceToHost, stream));
    run(hipStreamSynchronize(stream));
    if (e != hipSuccess) return SQ_ERR_HIP;
    int b = 0;
    for (int i = 1; i < n_alphas; ++i)
        if (mse[i] < mse[b]) b = i;
    *best = b;
    return SQ_OK;
}

}  // extern "C"
