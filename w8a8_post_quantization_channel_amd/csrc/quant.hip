// quant.hip -- the two quantization passes of the SmoothQuant W8A8 layer.
//
// quant_weight: offline fold W' = W diag(s) (kwkr.cn blog §3.2) and symmetric
//   int8 with one scale per output row (ADR-010 "Context" item 3). A block
//   spans whole rows with its threads owning fixed columns (their s values in
//   registers) and reduces R row maxima per barrier; the R rows stay in
//   registers between the max and the quantize pass, so W is read from HBM
//   exactly once.
// quant_act: runtime x * (1/s) strictly before the per-tensor quantizer
//   (kwkr.cn blog §3.2 and §5.2; ADR-010 "Key design" items 4-5). A lane owns
//   one 16-byte column vector and keeps its inv_s values in registers while
//   the four waves of a block walk interleaved rows.
//
// The weight pass works on "groups" of 16 consecutive elements of a row (32
// bytes of bf16, 64 of fp32), which become 16 int8 codes: one 16-byte store.
#include <algorithm>

#include "sq_device.h"
#include "sq_kernels.h"

namespace {

using sqd::u32x4;

template <int EB>
struct Group {
    static constexpr int V = EB;  // 16-byte vectors per 16-element group
    u32x4 v[V];
    __device__ __forceinline__ void load(const u32x4* p) {
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = __builtin_nontemporal_load(p + i);
    }
    __device__ __forceinline__ void widen(float (&e)[16]) const {
        constexpr int E = 16 / EB;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float t[E];
            sqd::unpack16<E>(v[i], t);
#pragma unroll
            for (int j = 0; j < E; ++j) e[i * E + j] = t[j];
        }
    }
};

// 16 consecutive fp32 values (64-byte aligned)
__device__ __forceinline__ void load16f(const float* __restrict__ p, float (&v)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4 t = ((const u32x4*)p)[q];
        v[4 * q + 0] = __uint_as_float(t.x);
        v[4 * q + 1] = __uint_as_float(t.y);
        v[4 * q + 2] = __uint_as_float(t.z);
        v[4 * q + 3] = __uint_as_float(t.w);
    }
}

__device__ __forceinline__ void store16(int8_t* __restrict__ dst, const int (&q)[16]) {
    u32x4 o;
    o.x = sqd::pack4_i8(q[0], q[1], q[2], q[3]);
    o.y = sqd::pack4_i8(q[4], q[5], q[6], q[7]);
    o.z = sqd::pack4_i8(q[8], q[9], q[10], q[11]);
    o.w = sqd::pack4_i8(q[12], q[13], q[14], q[15]);
    *(u32x4*)dst = o;
}

// Thread t of a block owns groups t, t + T, ... (GPL of them; T <= MAXT
// threads), so every wave load is one contiguous run of the row. R rows per
// iteration.
template <int EB, int GPL, int R, int MAXT>
__global__ __launch_bounds__(MAXT) void quant_weight_kernel(const u32x4* __restrict__ w, int64_t n, int64_t kgroups,
                                                            const float* __restrict__ s, int8_t* __restrict__ wq,
                                                            float* __restrict__ w_scale) {
    constexpr int VG = Group<EB>::V;
    __shared__ float red[2][16][R];  // [parity][wave][row]
    const int T = blockDim.x, nw = T >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float sv[GPL][16];
    bool own[GPL];
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
        const int64_t gi = threadIdx.x + (int64_t)g * T;
        own[g] = gi < kgroups;
        if (own[g]) load16f(s + gi * 16, sv[g]);
    }
    int parity = 0;
    for (int64_t r0 = (int64_t)blockIdx.x * R; r0 < n; r0 += (int64_t)gridDim.x * R, parity ^= 1) {
        Group<EB> raw[R][GPL];
        float mx[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int g = 0; g < GPL; ++g)
                if (own[g] && r0 + r < n) raw[r][g].load(w + ((r0 + r) * kgroups + threadIdx.x + (int64_t)g * T) * VG);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            mx[r] = 0.0f;
#pragma unroll
            for (int g = 0; g < GPL; ++g)
                if (own[g] && r0 + r < n) {
                    float e[16];
                    raw[r][g].widen(e);
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        mx[r] = __builtin_fmaxf(mx[r], __builtin_fabsf(__fmul_rn(e[j], sv[g][j])));
                }
            mx[r] = sqd::wave_max(mx[r]);
            if (lane == 0) red[parity][wave][r] = mx[r];
        }
        // one barrier per R rows: the buffer of the other parity is written
        // again only after the next barrier, when every thread has read it
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float m = red[parity][0][r];
            for (int i = 1; i < nw; ++i) m = __builtin_fmaxf(m, red[parity][i][r]);
            mx[r] = __builtin_fmaxf(m, sqd::kFloor);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r0 + r >= n) continue;
            const float ws = __fdiv_rn(mx[r], sqd::kQmax);
            const float inv_ws = __fdiv_rn(1.0f, ws);
#pragma unroll
            for (int g = 0; g < GPL; ++g)
                if (own[g]) {
                    float e[16];
                    int q[16];
                    raw[r][g].widen(e);
#pragma unroll
                    for (int j = 0; j < 16; ++j) q[j] = sqd::q8(__fmul_rn(__fmul_rn(e[j], sv[g][j]), inv_ws));
                    store16(wq + ((r0 + r) * kgroups + threadIdx.x + (int64_t)g * T) * 16, q);
                }
            if (threadIdx.x == 0) w_scale[r0 + r] = ws;
        }
    }
}

// Rows longer than 4096 groups (k > 65536): one block per row, the row is
// read twice and s is read from cache.
template <int EB>
__global__ __launch_bounds__(256) void quant_weight_long_kernel(const u32x4* __restrict__ w, int64_t kgroups,
                                                                const float* __restrict__ s,
                                                                int8_t* __restrict__ wq, float* __restrict__ w_scale) {
    constexpr int VG = Group<EB>::V;
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    float mx = 0.0f;
    for (int64_t gi = threadIdx.x; gi < kgroups; gi += 256) {
        Group<EB> raw;
        float e[16], sv[16];
        raw.load(w + (row * kgroups + gi) * VG);
        raw.widen(e);
        load16f(s + gi * 16, sv);
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(__fmul_rn(e[j], sv[j])));
    }
    mx = __builtin_fmaxf(sqd::block_max<4>(mx, red), sqd::kFloor);
    const float ws = __fdiv_rn(mx, sqd::kQmax);
    const float inv_ws = __fdiv_rn(1.0f, ws);
    for (int64_t gi = threadIdx.x; gi < kgroups; gi += 256) {
        Group<EB> raw;
        float e[16], sv[16];
        int q[16];
        raw.load(w + (row * kgroups + gi) * VG);
        raw.widen(e);
        load16f(s + gi * 16, sv);
#pragma unroll
        for (int j = 0; j < 16; ++j) q[j] = sqd::q8(__fmul_rn(__fmul_rn(e[j], sv[j]), inv_ws));
        store16(wq + (row * kgroups + gi) * 16, q);
    }
    if (threadIdx.x == 0) w_scale[row] = ws;
}

constexpr int kActThreads = 256;
constexpr int kActUnroll = 4;

// E int8 codes (E = 8: two dwords, E = 4: one dword)
template <int E>
__device__ __forceinline__ void store_codes(int8_t* __restrict__ dst, const int (&q)[E]) {
    if constexpr (E == 8) {
        sqd::u32x2 o;
        o.x = sqd::pack4_i8(q[0], q[1], q[2], q[3]);
        o.y = sqd::pack4_i8(q[4], q[5], q[6], q[7]);
        *(sqd::u32x2*)dst = o;
    } else {
        *(uint32_t*)dst = sqd::pack4_i8(q[0], q[1], q[2], q[3]);
    }
}

// A lane owns one 16-byte column vector (E = 16 / EB elements) of the input
// and keeps its E inv_s values in registers; the four waves of a block walk
// interleaved rows, so each wave instruction moves one contiguous 1 KB run.
template <int EB>
__global__ __launch_bounds__(kActThreads) void quant_act_kernel(const u32x4* __restrict__ x, int64_t rows,
                                                                int64_t kvec, int64_t rows_per_block,
                                                                const float* __restrict__ inv_s,
                                                                const float* __restrict__ act_scale,
                                                                int8_t* __restrict__ xq) {
    constexpr int E = 16 / EB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t v = (int64_t)blockIdx.x * 64 + lane;
    if (v >= kvec) return;  // no block-level synchronisation below
    float is[E];
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
        const u32x4 t = ((const u32x4*)(inv_s + v * E))[h];
        is[4 * h + 0] = __uint_as_float(t.x);
        is[4 * h + 1] = __uint_as_float(t.y);
        is[4 * h + 2] = __uint_as_float(t.z);
        is[4 * h + 3] = __uint_as_float(t.w);
    }
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

int device_cus() {
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

template <int EB, int GPL, int MAXT>
hipError_t launch_qw(const void* w, int64_t n, int64_t kgroups, const float* s, int8_t* wq, float* w_scale,
                     hipStream_t stream) {
    // rows per iteration: about 8 bf16 (4 fp32) group loads in flight per thread
    constexpr int R = ((EB == 2 ? 8 : 4) / GPL) > 0 ? (EB == 2 ? 8 : 4) / GPL : 1;
    const int64_t lanes = (kgroups + GPL - 1) / GPL;
    const int threads = (int)((lanes + 63) / 64 * 64);
    const int64_t row_groups = (n + R - 1) / R;
    const int64_t blocks = std::min<int64_t>(row_groups, (int64_t)device_cus() * 8);
    quant_weight_kernel<EB, GPL, R, MAXT><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
        (const u32x4*)w, n, kgroups, s, wq, w_scale);
    return hipGetLastError();
}

template <int EB>
hipError_t quant_weight_t(const void* w, int64_t n, int64_t k, const float* s, int8_t* wq, float* w_scale,
                          hipStream_t stream) {
    const int64_t kgroups = k / 16;
    // one group per thread in blocks of up to 1024 threads (128 VGPRs each);
    // longer rows: 512-thread blocks with 4 or 8 groups per thread
    if (kgroups <= 1024) return launch_qw<EB, 1, 1024>(w, n, kgroups, s, wq, w_scale, stream);
    if (kgroups <= 2048) return launch_qw<EB, 4, 512>(w, n, kgroups, s, wq, w_scale, stream);
    if (kgroups <= 4096) return launch_qw<EB, 8, 512>(w, n, kgroups, s, wq, w_scale, stream);
    quant_weight_long_kernel<EB><<<dim3((unsigned)n), dim3(256), 0, stream>>>((const u32x4*)w, kgroups, s, wq,
                                                                            w_scale);
    return hipGetLastError();
}

}  // namespace

namespace sqk {

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
    const dim3 grid((unsigned)strips, (unsigned)chunks), block(kActThreads);
    if (eb == 2)
        quant_act_kernel<2><<<grid, block, 0, stream>>>((const u32x4*)x, m, kvec, rpb, inv_s, act_scale, xq);
    else
        quant_act_kernel<4><<<grid, block, 0, stream>>>((const u32x4*)x, m, kvec, rpb, inv_s, act_scale, xq);
    return hipGetLastError();
}

}  // namespace sqk
