// quant.hip -- the two quantization passes of the SmoothQuant W8A8 layer.
//
// quant_weight: offline fold W' = W diag(s) (kwkr.cn blog §3.2) and symmetric
//   int8 with one scale per output row (ADR-010 "Context" item 3). One block of
//   256 threads owns one weight row; the row stays in registers between the
//   max pass and the quantize pass, so W is read from HBM exactly once.
// quant_act: runtime x * (1/s) strictly before the per-tensor quantizer
//   (kwkr.cn blog §3.2 and §5.2; ADR-010 "Key design" items 4-5). A lane owns
//   one 16-byte column vector and keeps its inv_s values in registers while the
//   four waves of a block walk interleaved rows; each wave moves one coalesced
//   row segment per step.
#include <algorithm>

#include "sq_device.h"
#include "sq_kernels.h"

namespace {

using sqd::u32x2;
using sqd::u32x4;

constexpr int kThreads = 256;

// load E consecutive fp32 values (E = 4 or 8, 16-byte aligned)
template <int E>
__device__ __forceinline__ void load_f32(const float* __restrict__ p, float (&v)[E]) {
    const u32x4* q = (const u32x4*)p;
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
        u32x4 t = q[h];
        v[4 * h + 0] = __uint_as_float(t.x);
        v[4 * h + 1] = __uint_as_float(t.y);
        v[4 * h + 2] = __uint_as_float(t.z);
        v[4 * h + 3] = __uint_as_float(t.w);
    }
}

// store E int8 codes (E = 4: one dword, E = 8: two dwords)
template <int E>
__device__ __forceinline__ void store_codes(int8_t* __restrict__ dst, const int (&q)[E]) {
    if constexpr (E == 8) {
        u32x2 o;
        o.x = sqd::pack4_i8(q[0], q[1], q[2], q[3]);
        o.y = sqd::pack4_i8(q[4], q[5], q[6], q[7]);
        *(u32x2*)dst = o;
    } else {
        *(uint32_t*)dst = sqd::pack4_i8(q[0], q[1], q[2], q[3]);
    }
}

// VPT > 0: the row is held in VPT registers-vectors per thread (kvec <= 256*VPT).
// VPT == 0: rows too long for registers; the row is read twice.
template <int EB, int VPT>
__global__ __launch_bounds__(kThreads) void quant_weight_kernel(const u32x4* __restrict__ w, int64_t kvec,
                                                                const float* __restrict__ s,
                                                                int8_t* __restrict__ wq,
                                                                float* __restrict__ w_scale) {
    constexpr int E = 16 / EB;
    __shared__ float red[kThreads / 64];
    const int64_t row = blockIdx.x;
    const u32x4* wr = w + row * kvec;
    int8_t* qr = wq + row * kvec * E;
    float mx = 0.0f;
    constexpr int R = VPT > 0 ? VPT : 1;
    u32x4 raw[R];
    if constexpr (VPT > 0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t v = threadIdx.x + (int64_t)i * kThreads;
            if (v < kvec) raw[i] = __builtin_nontemporal_load(wr + v);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t v = threadIdx.x + (int64_t)i * kThreads;
            if (v < kvec) {
                float e[E], sv[E];
                sqd::unpack16<E>(raw[i], e);
                load_f32<E>(s + v * E, sv);
#pragma unroll
                for (int t = 0; t < E; ++t) mx = __builtin_fmaxf(mx, __builtin_fabsf(__fmul_rn(e[t], sv[t])));
            }
        }
    } else {
        for (int64_t v = threadIdx.x; v < kvec; v += kThreads) {
            float e[E], sv[E];
            sqd::unpack16<E>(wr[v], e);
            load_f32<E>(s + v * E, sv);
#pragma unroll
            for (int t = 0; t < E; ++t) mx = __builtin_fmaxf(mx, __builtin_fabsf(__fmul_rn(e[t], sv[t])));
        }
    }
    mx = sqd::block_max<kThreads / 64>(mx, red);
    mx = __builtin_fmaxf(mx, sqd::kFloor);
    const float ws = __fdiv_rn(mx, sqd::kQmax);
    const float inv_ws = __fdiv_rn(1.0f, ws);
    auto quantize_vec = [&](const u32x4& r, int64_t v) {
        float e[E], sv[E];
        int q[E];
        sqd::unpack16<E>(r, e);
        load_f32<E>(s + v * E, sv);
#pragma unroll
        for (int t = 0; t < E; ++t) q[t] = sqd::q8(__fmul_rn(__fmul_rn(e[t], sv[t]), inv_ws));
        store_codes<E>(qr + v * E, q);
    };
    if constexpr (VPT > 0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t v = threadIdx.x + (int64_t)i * kThreads;
            if (v < kvec) quantize_vec(raw[i], v);
        }
    } else {
        for (int64_t v = threadIdx.x; v < kvec; v += kThreads) quantize_vec(wr[v], v);
    }
    if (threadIdx.x == 0) w_scale[row] = ws;
}

constexpr int kActUnroll = 4;

template <int EB>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const u32x4* __restrict__ x, int64_t rows,
                                                             int64_t kvec, int64_t rows_per_block,
                                                             const float* __restrict__ inv_s,
                                                             const float* __restrict__ act_scale,
                                                             int8_t* __restrict__ xq) {
    constexpr int E = 16 / EB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t v = (int64_t)blockIdx.x * 64 + lane;
    if (v >= kvec) return;  // no block-level synchronisation below
    float is[E];
    load_f32<E>(inv_s + v * E, is);
    const float inv_a = __fdiv_rn(1.0f, act_scale[0]);
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = min(rows, r0 + rows_per_block);
    auto quantize = [&](const u32x4& raw, int64_t r) {
        float e[E];
        int q[E];
        sqd::unpack16<E>(raw, e);
#pragma unroll
        for (int t = 0; t < E; ++t) q[t] = sqd::q8(__fmul_rn(__fmul_rn(e[t], is[t]), inv_a));
        store_codes<E>(xq + (r * kvec + v) * E, q);
    };
    int64_t r = r0 + wave;
    for (; r + 4 * (kActUnroll - 1) < r1; r += 4 * kActUnroll) {
        u32x4 t[kActUnroll];
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) t[u] = __builtin_nontemporal_load(x + (r + 4 * u) * kvec + v);
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) quantize(t[u], r + 4 * u);
    }
    for (; r < r1; r += 4) quantize(__builtin_nontemporal_load(x + r * kvec + v), r);
}

}  // namespace

namespace sqk {

hipError_t quant_weight(const void* w, int wt, int64_t n, int64_t k, const float* s, int8_t* wq,
                        float* w_scale, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int eb = elem_bytes(wt);
    const int64_t kvec = k * eb / 16;
    const int64_t per_thread = (kvec + kThreads - 1) / kThreads;
    const dim3 grid((unsigned)n), block(kThreads);
    const u32x4* wv = (const u32x4*)w;
#define SQ_QW(EBV, VPTV) quant_weight_kernel<EBV, VPTV><<<grid, block, 0, stream>>>(wv, kvec, s, wq, w_scale)
    if (eb == 2) {
        if (per_thread <= 1) SQ_QW(2, 1);
        else if (per_thread <= 2) SQ_QW(2, 2);
        else if (per_thread <= 4) SQ_QW(2, 4);
        else if (per_thread <= 8) SQ_QW(2, 8);
        else if (per_thread <= 16) SQ_QW(2, 16);
        else SQ_QW(2, 0);
    } else {
        if (per_thread <= 1) SQ_QW(4, 1);
        else if (per_thread <= 2) SQ_QW(4, 2);
        else if (per_thread <= 4) SQ_QW(4, 4);
        else if (per_thread <= 8) SQ_QW(4, 8);
        else if (per_thread <= 16) SQ_QW(4, 16);
        else SQ_QW(4, 0);
    }
#undef SQ_QW
    return hipGetLastError();
}

hipError_t quant_act(const void* x, int xt, int64_t m, int64_t k, const float* inv_s, const float* act_scale,
                     int8_t* xq, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    const int eb = elem_bytes(xt);
    const int64_t kvec = k * eb / 16;
    const int64_t strips = (kvec + 63) / 64;
    const int64_t granule = 4 * kActUnroll;
    int64_t target_chunks = std::max<int64_t>(1, 4096 / strips);
    int64_t rpb = (m + target_chunks - 1) / target_chunks;
    rpb = std::max<int64_t>(granule, (rpb + granule - 1) / granule * granule);
    int64_t chunks = (m + rpb - 1) / rpb;
    if (chunks > 65535) {
        rpb = (m + 65534) / 65535;
        rpb = (rpb + granule - 1) / granule * granule;
        chunks = (m + rpb - 1) / rpb;
    }
    const dim3 grid((unsigned)strips, (unsigned)chunks), block(kThreads);
    if (eb == 2)
        quant_act_kernel<2><<<grid, block, 0, stream>>>((const u32x4*)x, m, kvec, rpb, inv_s, act_scale, xq);
    else
        quant_act_kernel<4><<<grid, block, 0, stream>>>((const u32x4*)x, m, kvec, rpb, inv_s, act_scale, xq);
    return hipGetLastError();
}

}  // namespace sqk
