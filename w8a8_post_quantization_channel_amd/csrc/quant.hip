// quant.hip -- the two quantization passes of the SmoothQuant W8A8 layer.
//
// quant_weight: offline fold W' = W diag(s) (kwkr.cn blog §3.2) and symmetric
//   int8 with one scale per output row (ADR-010 "Context" item 3). One to four
//   waves own one weight row; the row stays in registers between the max pass
//   and the quantize pass, so W is read from HBM exactly once (rows longer than
//   16 K bf16 values per wave group fall back to reading the row twice).
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

// Register-resident rows: a group of WPR waves owns one row (4 / WPR rows per
// block); lane l of wave g of the group holds vectors g*64 + l + i*64*WPR,
// i < VPT, so the row is read from HBM once and every lane has VPT 16-byte
// loads in flight.
template <int EB, int WPR, int VPT>
__global__ __launch_bounds__(kThreads) void quant_weight_rows_kernel(const u32x4* __restrict__ w, int64_t n,
                                                                     int64_t kvec, const float* __restrict__ s,
                                                                     int8_t* __restrict__ wq,
                                                                     float* __restrict__ w_scale) {
    constexpr int E = 16 / EB;
    constexpr int RPB = 4 / WPR;
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const int sub = wave % WPR;
    const bool live = row < n;
    const u32x4* wr = w + row * kvec;
    u32x4 raw[VPT];
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t v = sub * 64 + lane + (int64_t)i * 64 * WPR;
        if (live && v < kvec) raw[i] = __builtin_nontemporal_load(wr + v);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t v = sub * 64 + lane + (int64_t)i * 64 * WPR;
        if (live && v < kvec) {
            float e[E], sv[E];
            sqd::unpack16<E>(raw[i], e);
            load_f32<E>(s + v * E, sv);
#pragma unroll
            for (int t = 0; t < E; ++t) mx = __builtin_fmaxf(mx, __builtin_fabsf(__fmul_rn(e[t], sv[t])));
        }
    }
    mx = sqd::wave_max(mx);
    if constexpr (WPR > 1) {
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        const int g0 = (wave / WPR) * WPR;
        mx = red[g0];
#pragma unroll
        for (int i = 1; i < WPR; ++i) mx = __builtin_fmaxf(mx, red[g0 + i]);
    }
    if (!live) return;  // no barrier follows
    mx = __builtin_fmaxf(mx, sqd::kFloor);
    const float ws = __fdiv_rn(mx, sqd::kQmax);
    const float inv_ws = __fdiv_rn(1.0f, ws);
    int8_t* qr = wq + row * kvec * E;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t v = sub * 64 + lane + (int64_t)i * 64 * WPR;
        if (v < kvec) {
            float e[E], sv[E];
            int q[E];
            sqd::unpack16<E>(raw[i], e);
            load_f32<E>(s + v * E, sv);
#pragma unroll
            for (int t = 0; t < E; ++t) q[t] = sqd::q8(__fmul_rn(__fmul_rn(e[t], sv[t]), inv_ws));
            store_codes<E>(qr + v * E, q);
        }
    }
    if (sub == 0 && lane == 0) w_scale[row] = ws;
}

// Rows too long for registers: one block per row, the row is read twice.
template <int EB>
__global__ __launch_bounds__(kThreads) void quant_weight_stream_kernel(const u32x4* __restrict__ w, int64_t kvec,
                                                                       const float* __restrict__ s,
                                                                       int8_t* __restrict__ wq,
                                                                       float* __restrict__ w_scale) {
    constexpr int E = 16 / EB;
    __shared__ float red[kThreads / 64];
    const int64_t row = blockIdx.x;
    const u32x4* wr = w + row * kvec;
    int8_t* qr = wq + row * kvec * E;
    float mx = 0.0f;
    for (int64_t v = threadIdx.x; v < kvec; v += kThreads) {
        float e[E], sv[E];
        sqd::unpack16<E>(wr[v], e);
        load_f32<E>(s + v * E, sv);
#pragma unroll
        for (int t = 0; t < E; ++t) mx = __builtin_fmaxf(mx, __builtin_fabsf(__fmul_rn(e[t], sv[t])));
    }
    mx = sqd::block_max<kThreads / 64>(mx, red);
    mx = __builtin_fmaxf(mx, sqd::kFloor);
    const float ws = __fdiv_rn(mx, sqd::kQmax);
    const float inv_ws = __fdiv_rn(1.0f, ws);
    for (int64_t v = threadIdx.x; v < kvec; v += kThreads) {
        float e[E], sv[E];
        int q[E];
        sqd::unpack16<E>(wr[v], e);
        load_f32<E>(s + v * E, sv);
#pragma unroll
        for (int t = 0; t < E; ++t) q[t] = sqd::q8(__fmul_rn(__fmul_rn(e[t], sv[t]), inv_ws));
        store_codes<E>(qr + v * E, q);
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

template <int EB, int WPR>
hipError_t launch_rows(const u32x4* w, int64_t n, int64_t kvec, const float* s, int8_t* wq, float* w_scale,
                       int64_t per_lane, hipStream_t stream) {
    const dim3 grid((unsigned)((n + 4 / WPR - 1) / (4 / WPR))), block(kThreads);
    if (per_lane <= 2)
        quant_weight_rows_kernel<EB, WPR, 2><<<grid, block, 0, stream>>>(w, n, kvec, s, wq, w_scale);
    else if (per_lane <= 4)
        quant_weight_rows_kernel<EB, WPR, 4><<<grid, block, 0, stream>>>(w, n, kvec, s, wq, w_scale);
    else if (per_lane <= 8)
        quant_weight_rows_kernel<EB, WPR, 8><<<grid, block, 0, stream>>>(w, n, kvec, s, wq, w_scale);
    else if (per_lane <= 12)
        quant_weight_rows_kernel<EB, WPR, 12><<<grid, block, 0, stream>>>(w, n, kvec, s, wq, w_scale);
    else
        quant_weight_rows_kernel<EB, WPR, 16><<<grid, block, 0, stream>>>(w, n, kvec, s, wq, w_scale);
    return hipGetLastError();
}

template <int EB>
hipError_t quant_weight_t(const void* w, int64_t n, int64_t k, const float* s, int8_t* wq, float* w_scale,
                          hipStream_t stream) {
    const int64_t kvec = k * EB / 16;
    const u32x4* wv = (const u32x4*)w;
    // fewest waves per row that keep at most 16 vectors per lane
    for (int wpr : {1, 2, 4}) {
        const int64_t per_lane = (kvec + 64 * wpr - 1) / (64 * wpr);
        if (per_lane > 16) continue;
        if (wpr == 1) return launch_rows<EB, 1>(wv, n, kvec, s, wq, w_scale, per_lane, stream);
        if (wpr == 2) return launch_rows<EB, 2>(wv, n, kvec, s, wq, w_scale, per_lane, stream);
        return launch_rows<EB, 4>(wv, n, kvec, s, wq, w_scale, per_lane, stream);
    }
    quant_weight_stream_kernel<EB><<<dim3((unsigned)n), dim3(kThreads), 0, stream>>>(wv, kvec, s, wq, w_scale);
    return hipGetLastError();
}

hipError_t quant_weight(const void* w, int wt, int64_t n, int64_t k, const float* s, int8_t* wq,
                        float* w_scale, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    return elem_bytes(wt) == 2 ? quant_weight_t<2>(w, n, k, s, wq, w_scale, stream)
                               : quant_weight_t<4>(w, n, k, s, wq, w_scale, stream);
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
