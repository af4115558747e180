// norm.hip -- RMSNorm in front of a smoothed projection, with 1/s folded into
// the norm weight so the norm's output is already X/s and goes straight into
// the per-tensor quantizer (kwkr.cn blog §2.3 and §3.2: the per-channel 1/s is
// absorbed by the gamma of the preceding norm, once, offline, and the scaling
// still happens before the rounding).
//
// The row's sum of squares is taken in fp64 (squares of bf16 or fp32 values
// are exact in fp64, so only the order of the additions is free) and
// r = fp32(1 / sqrt(sum / k + eps)) is evaluated in fp64 and rounded once.
// A block of 256 threads takes one to eight rows, held in registers between
// the reduction and the output pass up to 256 * 8 16-byte vectors per row
// (16384 bf16 or 8192 fp32 values); longer rows are read a second time
// (from L2).
#include <algorithm>
#include <type_traits>

#include "sq_device.h"
#include "sq_kernels.h"

namespace {

using sqd::u32x4;

constexpr int kNormThreads = 256;
constexpr int kNormWaves = kNormThreads / 64;

enum NormOut { kOutF32, kOutBF16, kOutI8 };

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// 16 bytes -> E values widened to fp32
template <int E>
__device__ __forceinline__ void widen(const u32x4& v, float (&e)[E]) {
    sqd::unpack16<E>(v, e);
}

template <int E>
__device__ __forceinline__ double sum_sq(const u32x4& v) {
    float e[E];
    widen<E>(v, e);
    // d * d is exact in fp64 (at most 48 significant bits), so the fused
    // multiply-add rounds exactly where a product followed by a sum would
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const double d = (double)e[i];
        s = __fma_rn(d, d, s);
    }
    return s;
}

// gamma[c * E .. c * E + E - 1] (16-byte aligned fp32)
template <int E>
__device__ __forceinline__ void load_gamma(const float* __restrict__ g, int64_t c, float (&out)[E]) {
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
        const u32x4 t = ((const u32x4*)(g + c * E))[q];
        out[4 * q + 0] = __uint_as_float(t.x);
        out[4 * q + 1] = __uint_as_float(t.y);
        out[4 * q + 2] = __uint_as_float(t.z);
        out[4 * q + 3] = __uint_as_float(t.w);
    }
}

// One output vector: E values of y = fl(fl(h r) gamma) stored as fp32 or
// bf16, or E int8 codes of fl(y inv_a) (round half to even, clamp).
template <int E, NormOut OUT>
__device__ __forceinline__ void emit(const u32x4& v, float r, const float (&g)[E], float inv_a, void* out,
                                     int64_t idx) {
    float e[E];
    widen<E>(v, e);
    float y[E];
#pragma unroll
    for (int i = 0; i < E; ++i) y[i] = __fmul_rn(__fmul_rn(e[i], r), g[i]);
    if constexpr (OUT == kOutF32) {
#pragma unroll
        for (int q = 0; q < E / 4; ++q)
            *(u32x4*)((float*)out + idx + 4 * q) = u32x4{__float_as_uint(y[4 * q]), __float_as_uint(y[4 * q + 1]),
                                                         __float_as_uint(y[4 * q + 2]), __float_as_uint(y[4 * q + 3])};
    } else if constexpr (OUT == kOutBF16) {
        uint32_t w[E / 2];
#pragma unroll
        for (int i = 0; i < E / 2; ++i)
            w[i] = sqd::f32_to_bf16_bits(y[2 * i]) | (sqd::f32_to_bf16_bits(y[2 * i + 1]) << 16);
        if constexpr (E == 8)
            *(u32x4*)((uint16_t*)out + idx) = u32x4{w[0], w[1], w[2], w[3]};
        else
            *(sqd::u32x2*)((uint16_t*)out + idx) = sqd::u32x2{w[0], w[1]};
    } else {
        // clamp to [-127, 127], then round half to even with the fp32 adder:
        // for |v| < 2^22, fl(v + 1.5 * 2^23) = rint(v) + 1.5 * 2^23 and the low
        // byte of its bits is rint(v) as an int8 (rint and the integer-bounded
        // clamp commute, so this equals clamp(rint(v)))
        uint32_t b[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float v = __builtin_fminf(__builtin_fmaxf(__fmul_rn(y[i], inv_a), -sqd::kQmax), sqd::kQmax);
            b[i] = __float_as_uint(__fadd_rn(v, 12582912.0f));
        }
        uint32_t w[E / 4];
#pragma unroll
        for (int d = 0; d < E / 4; ++d) {
            const uint32_t lo = __builtin_amdgcn_perm(b[4 * d + 1], b[4 * d], 0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm(b[4 * d + 3], b[4 * d + 2], 0x0c0c0400u);
            w[d] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        if constexpr (E == 8)
            *(sqd::u32x2*)((int8_t*)out + idx) = sqd::u32x2{w[0], w[1]};
        else
            *(uint32_t*)((int8_t*)out + idx) = w[0];
    }
}

// One block of 256 threads takes R consecutive rows. VPT > 0: each row is
// held in VPT vectors per thread (kvec <= 256 * VPT), all R rows loaded
// before the reduction so R * VPT 16-byte loads per thread are in flight.
// VPT == 0 (R = 1): the row is streamed twice.
template <int EB, int VPT, int R, NormOut OUT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const u32x4* __restrict__ h, int64_t m, int64_t kvec,
                                                               int64_t k, const float* __restrict__ gamma, float eps,
                                                               const float* __restrict__ act_scale,
                                                               void* __restrict__ out, float* __restrict__ r_out) {
    constexpr int E = 16 / EB;
    static_assert(VPT > 0 || R == 1, "streamed rows go one per block");
    __shared__ double red[R][kNormWaves];
    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * R;

    double ss[R];
    u32x4 v[R][VPT > 0 ? VPT : 1];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        ss[q] = 0.0;
        const int64_t row = row0 + q;
        const u32x4* hr = h + (row < m ? row : 0) * kvec;
        if constexpr (VPT > 0) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t c = tid + (int64_t)i * kNormThreads;
                v[q][i] = (row < m && c < kvec) ? __builtin_nontemporal_load(hr + c) : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
            for (int64_t c = tid; c < kvec; c += kNormThreads) ss[q] += sum_sq<E>(hr[c]);
        }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
        if constexpr (VPT > 0) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) ss[q] += sum_sq<E>(v[q][i]);
        }
        ss[q] = wave_sum_f64(ss[q]);
        if ((tid & 63) == 0) red[q][tid >> 6] = ss[q];
    }
    __syncthreads();
    const float inv_a = OUT == kOutI8 ? __fdiv_rn(1.0f, act_scale[0]) : 0.0f;
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int64_t row = row0 + q;
        if (row >= m) break;
        double total = red[q][0];
#pragma unroll
        for (int w = 1; w < kNormWaves; ++w) total += red[q][w];
        const float r = (float)(1.0 / sqrt(total / (double)k + (double)eps));
        if (r_out && tid == 0) r_out[row] = r;
        if constexpr (VPT > 0) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t c = tid + (int64_t)i * kNormThreads;
                if (c < kvec) {
                    float g[E];
                    load_gamma<E>(gamma, c, g);
                    emit<E, OUT>(v[q][i], r, g, inv_a, out, row * k + c * E);
                }
            }
        } else {
            const u32x4* hr = h + row * kvec;
            for (int64_t c = tid; c < kvec; c += kNormThreads) {
                float g[E];
                load_gamma<E>(gamma, c, g);
                emit<E, OUT>(hr[c], r, g, inv_a, out, row * k + c * E);
            }
        }
    }
}

// Persistent form of the register-resident kernel: a block walks groups of
// R rows g, g + grid, ... and issues the loads of its next group before it
// reduces and writes the current one, so every thread keeps R * VPT 16-byte
// loads in flight through the reduction, the barrier and the stores. A
// thread's columns are the same in every row, so their weights are loaded
// once (reloading them per row costs more load traffic than the row itself).
// The LDS partials alternate between two buffers: one barrier per group.
template <int EB, int VPT, int R, NormOut OUT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_stream_kernel(const u32x4* __restrict__ h, int64_t m,
                                                                      int64_t kvec, int64_t k,
                                                                      const float* __restrict__ gamma, float eps,
                                                                      const float* __restrict__ act_scale,
                                                                      void* __restrict__ out,
                                                                      float* __restrict__ r_out) {
    constexpr int E = 16 / EB;
    static_assert(VPT > 0, "register-resident rows only");
    __shared__ double red[2][R][kNormWaves];
    const int tid = threadIdx.x;
    const int64_t groups = (m + R - 1) / R;
    const float inv_a = OUT == kOutI8 ? __fdiv_rn(1.0f, act_scale[0]) : 0.0f;
    auto load = [&](int64_t g, u32x4 (&buf)[R][VPT]) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int64_t row = g * R + q;
            const bool ok = g < groups && row < m;
            const u32x4* hr = h + (ok ? row : 0) * kvec;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t c = tid + (int64_t)i * kNormThreads;
                buf[q][i] = (ok && c < kvec) ? __builtin_nontemporal_load(hr + c) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // the block's columns are the same for every row: their weights stay in registers
    float gm[VPT][E];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t c = tid + (int64_t)i * kNormThreads;
        if (c < kvec)
            load_gamma<E>(gamma, c, gm[i]);
        else
#pragma unroll
            for (int e = 0; e < E; ++e) gm[i][e] = 0.0f;
    }
    auto process = [&](int64_t g, const u32x4 (&buf)[R][VPT], int par) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            double ss = 0.0;
#pragma unroll
            for (int i = 0; i < VPT; ++i) ss += sum_sq<E>(buf[q][i]);
            ss = wave_sum_f64(ss);
            if ((tid & 63) == 0) red[par][q][tid >> 6] = ss;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int64_t row = g * R + q;
            if (row >= m) break;
            double total = red[par][q][0];
#pragma unroll
            for (int w = 1; w < kNormWaves; ++w) total += red[par][q][w];
            const float r = (float)(1.0 / sqrt(total / (double)k + (double)eps));
            if (r_out && tid == 0) r_out[row] = r;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t c = tid + (int64_t)i * kNormThreads;
                if (c < kvec) emit<E, OUT>(buf[q][i], r, gm[i], inv_a, out, row * k + c * E);
            }
        }
    };
    u32x4 a[R][VPT], b[R][VPT];
    const int64_t step = gridDim.x;
    int64_t g = blockIdx.x;
    load(g, a);
    // groups in pairs: the loads of the next group go out before each group is processed
    for (; g < groups; g += 2 * step) {
        load(g + step, b);
        process(g, a, 0);
        if (g + step >= groups) break;
        load(g + 2 * step, a);
        process(g + step, b, 1);
    }
}

// Several consumers of one norm output (q, k and v after the attention norm;
// gate and up after the MLP norm), each with its own folded weight and act
// scale: the row is read and reduced once, fl(h r) formed once per element,
// and every consumer's codes written from it exactly as the single-consumer
// pass writes them. The consumers' weights stay in registers (NC x VPT x E).
constexpr int kNormMaxConsumers = 4;
struct NormConsumers {
    const float* gamma[kNormMaxConsumers];
    const float* act_scale[kNormMaxConsumers];
    int8_t* xq[kNormMaxConsumers];
};

template <int EB, int VPT, int R, int NC>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_multi_kernel(const u32x4* __restrict__ h, int64_t m,
                                                                     int64_t kvec, int64_t k, float eps,
                                                                     const NormConsumers cons,
                                                                     float* __restrict__ r_out) {
    constexpr int E = 16 / EB;
    __shared__ double red[2][R][kNormWaves];
    const int tid = threadIdx.x;
    const int64_t groups = (m + R - 1) / R;
    float inv_a[NC];
    float gm[NC][VPT][E];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        inv_a[c] = __fdiv_rn(1.0f, cons.act_scale[c][0]);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t v = tid + (int64_t)i * kNormThreads;
            if (v < kvec)
                load_gamma<E>(cons.gamma[c], v, gm[c][i]);
            else
#pragma unroll
                for (int e = 0; e < E; ++e) gm[c][i][e] = 0.0f;
        }
    }
    auto load = [&](int64_t g, u32x4 (&buf)[R][VPT]) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int64_t row = g * R + q;
            const bool ok = g < groups && row < m;
            const u32x4* hr = h + (ok ? row : 0) * kvec;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t v = tid + (int64_t)i * kNormThreads;
                buf[q][i] = (ok && v < kvec) ? __builtin_nontemporal_load(hr + v) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto process = [&](int64_t g, const u32x4 (&buf)[R][VPT], int par) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            double ss = 0.0;
#pragma unroll
            for (int i = 0; i < VPT; ++i) ss += sum_sq<E>(buf[q][i]);
            ss = wave_sum_f64(ss);
            if ((tid & 63) == 0) red[par][q][tid >> 6] = ss;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int64_t row = g * R + q;
            if (row >= m) break;
            double total = red[par][q][0];
#pragma unroll
            for (int w = 1; w < kNormWaves; ++w) total += red[par][q][w];
            const float r = (float)(1.0 / sqrt(total / (double)k + (double)eps));
            if (r_out && tid == 0) r_out[row] = r;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t v = tid + (int64_t)i * kNormThreads;
                if (v >= kvec) continue;
                float e[E], hr[E];
                widen<E>(buf[q][i], e);
#pragma unroll
                for (int j = 0; j < E; ++j) hr[j] = __fmul_rn(e[j], r);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    // as emit<E, kOutI8>: clamp, then round half to even with the fp32 adder
                    uint32_t b[E];
#pragma unroll
                    for (int j = 0; j < E; ++j) {
                        const float y = __fmul_rn(hr[j], gm[c][i][j]);
                        const float t = __builtin_fminf(__builtin_fmaxf(__fmul_rn(y, inv_a[c]), -sqd::kQmax), sqd::kQmax);
                        b[j] = __float_as_uint(__fadd_rn(t, 12582912.0f));
                    }
                    uint32_t w[E / 4];
#pragma unroll
                    for (int d = 0; d < E / 4; ++d) {
                        const uint32_t lo = __builtin_amdgcn_perm(b[4 * d + 1], b[4 * d], 0x0c0c0400u);
                        const uint32_t hi = __builtin_amdgcn_perm(b[4 * d + 3], b[4 * d + 2], 0x0c0c0400u);
                        w[d] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                    }
                    int8_t* dst = cons.xq[c] + row * k + v * E;
                    if constexpr (E == 8)
                        *(sqd::u32x2*)dst = sqd::u32x2{w[0], w[1]};
                    else
                        *(uint32_t*)dst = w[0];
                }
            }
        }
    };
    u32x4 a[R][VPT], b[R][VPT];
    const int64_t step = gridDim.x;
    int64_t g = blockIdx.x;
    load(g, a);
    for (; g < groups; g += 2 * step) {
        load(g + step, b);
        process(g, a, 0);
        if (g + step >= groups) break;
        load(g + 2 * step, a);
        process(g + step, b, 1);
    }
}

int norm_cus() {
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

template <int EB, int VPT, int R, NormOut OUT>
hipError_t launch_rows(const void* h, int64_t m, int64_t kvec, int64_t k, const float* gamma, float eps,
                       const float* act_scale, void* out, float* r_out, hipStream_t stream) {
    const int64_t groups = (m + R - 1) / R;
    if constexpr (VPT > 0) {
        // as many blocks as are resident at once (all groups dealt out evenly)
        static const int per_cu = [] {
            int b = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, rmsnorm_stream_kernel<EB, VPT, R, OUT>,
                                                             kNormThreads, 0) != hipSuccess || b < 1)
                b = 1;
            return b;
        }();
        const int64_t grid = std::min<int64_t>(groups, (int64_t)per_cu * norm_cus());
        rmsnorm_stream_kernel<EB, VPT, R, OUT><<<dim3((unsigned)grid), dim3(kNormThreads), 0, stream>>>(
            (const u32x4*)h, m, kvec, k, gamma, eps, act_scale, out, r_out);
    } else {
        rmsnorm_kernel<EB, VPT, R, OUT><<<dim3((unsigned)groups), dim3(kNormThreads), 0, stream>>>(
            (const u32x4*)h, m, kvec, k, gamma, eps, act_scale, out, r_out);
    }
    return hipGetLastError();
}

// rows per block so that about eight 16-byte loads per thread are in flight
template <int EB, NormOut OUT>
hipError_t launch_norm(const void* h, int64_t m, int64_t k, const float* gamma, float eps, const float* act_scale,
                       void* out, float* r_out, hipStream_t stream) {
    const int64_t kvec = k * EB / 16;
    const int64_t per = (kvec + kNormThreads - 1) / kNormThreads;  // vectors per thread per row
    switch (per) {
        case 1: return launch_rows<EB, 1, 8, OUT>(h, m, kvec, k, gamma, eps, act_scale, out, r_out, stream);
        case 2: return launch_rows<EB, 2, 4, OUT>(h, m, kvec, k, gamma, eps, act_scale, out, r_out, stream);
        case 3: return launch_rows<EB, 3, 2, OUT>(h, m, kvec, k, gamma, eps, act_scale, out, r_out, stream);
        case 4: return launch_rows<EB, 4, 2, OUT>(h, m, kvec, k, gamma, eps, act_scale, out, r_out, stream);
        case 5:
        case 6: return launch_rows<EB, 6, 1, OUT>(h, m, kvec, k, gamma, eps, act_scale, out, r_out, stream);
        case 7:
        case 8: return launch_rows<EB, 8, 1, OUT>(h, m, kvec, k, gamma, eps, act_scale, out, r_out, stream);
        default: return launch_rows<EB, 0, 1, OUT>(h, m, kvec, k, gamma, eps, act_scale, out, r_out, stream);
    }
}

template <int EB, int VPT, int R, int NC>
hipError_t launch_multi_rows(const void* h, int64_t m, int64_t kvec, int64_t k, float eps,
                             const NormConsumers& cons, float* r_out, hipStream_t stream) {
    static const int per_cu = [] {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, rmsnorm_multi_kernel<EB, VPT, R, NC>, kNormThreads, 0) !=
                hipSuccess ||
            b < 1)
            b = 1;
        return b;
    }();
    const int64_t groups = (m + R - 1) / R;
    const int64_t grid = std::min<int64_t>(groups, (int64_t)per_cu * norm_cus());
    rmsnorm_multi_kernel<EB, VPT, R, NC><<<dim3((unsigned)grid), dim3(kNormThreads), 0, stream>>>(
        (const u32x4*)h, m, kvec, k, eps, cons, r_out);
    return hipGetLastError();
}

// the single-consumer kernel's rows per block for the same row length; 0
// when the consumers' weights would not fit the registers (VPT x NC > 12)
template <int EB, int NC>
hipError_t launch_multi(const void* h, int64_t m, int64_t k, float eps, const NormConsumers& cons, float* r_out,
                        hipStream_t stream) {
    const int64_t kvec = k * EB / 16;
    const int64_t per = (kvec + kNormThreads - 1) / kNormThreads;
    if (per * NC > 12) return hipErrorInvalidValue;
    switch (per) {
        case 1: return launch_multi_rows<EB, 1, 8, NC>(h, m, kvec, k, eps, cons, r_out, stream);
        case 2: return launch_multi_rows<EB, 2, 4, NC>(h, m, kvec, k, eps, cons, r_out, stream);
        case 3: return launch_multi_rows<EB, 3, 2, NC>(h, m, kvec, k, eps, cons, r_out, stream);
        case 4: return launch_multi_rows<EB, 4, 2, NC>(h, m, kvec, k, eps, cons, r_out, stream);
        case 5:
        case 6: return launch_multi_rows<EB, 6, 1, NC>(h, m, kvec, k, eps, cons, r_out, stream);
        case 7:
        case 8: return launch_multi_rows<EB, 8, 1, NC>(h, m, kvec, k, eps, cons, r_out, stream);
    }
    return hipErrorInvalidValue;
}

template <int EB>
hipError_t launch_multi_n(int n, const void* h, int64_t m, int64_t k, float eps, const NormConsumers& cons,
                          float* r_out, hipStream_t stream) {
    switch (n) {
        case 2: return launch_multi<EB, 2>(h, m, k, eps, cons, r_out, stream);
        case 3: return launch_multi<EB, 3>(h, m, k, eps, cons, r_out, stream);
        case 4: return launch_multi<EB, 4>(h, m, k, eps, cons, r_out, stream);
    }
    return hipErrorInvalidValue;
}

// gamma_folded = fl(gamma * inv_s), one thread per channel
__global__ __launch_bounds__(256) void fold_kernel(const float* __restrict__ gamma, const float* __restrict__ inv_s,
                                                   int64_t k, float* __restrict__ out) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j < k) out[j] = __fmul_rn(gamma[j], inv_s[j]);
}

}  // namespace

namespace sqk {

hipError_t rmsnorm(const void* h, int ht, int64_t m, int64_t k, const float* gamma, float eps, void* y, int yt,
                   float* r_out, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    if (ht == kBF16)
        return yt == kBF16 ? launch_norm<2, kOutBF16>(h, m, k, gamma, eps, nullptr, y, r_out, stream)
                           : launch_norm<2, kOutF32>(h, m, k, gamma, eps, nullptr, y, r_out, stream);
    return yt == kBF16 ? launch_norm<4, kOutBF16>(h, m, k, gamma, eps, nullptr, y, r_out, stream)
                       : launch_norm<4, kOutF32>(h, m, k, gamma, eps, nullptr, y, r_out, stream);
}

hipError_t rmsnorm_quant(const void* h, int ht, int64_t m, int64_t k, const float* gamma_folded, float eps,
                         const float* act_scale, int8_t* xq, float* r_out, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    if (ht == kBF16) return launch_norm<2, kOutI8>(h, m, k, gamma_folded, eps, act_scale, xq, r_out, stream);
    return launch_norm<4, kOutI8>(h, m, k, gamma_folded, eps, act_scale, xq, r_out, stream);
}

hipError_t rmsnorm_quant_multi(const void* h, int ht, int64_t m, int64_t k, float eps, int n,
                               const float* const* gamma_folded, const float* const* act_scale, int8_t* const* xq,
                               float* r_out, hipStream_t stream) {
    if (m == 0 || n <= 0) return hipSuccess;
    if (n > kNormMaxConsumers) return hipErrorInvalidValue;
    const int64_t per = (k * elem_bytes(ht) / 16 + kNormThreads - 1) / kNormThreads;
    if (n == 1 || per * n > 12) {  // one pass per consumer (rows too long for all weights in registers)
        for (int c = 0; c < n; ++c) {
            const hipError_t e = rmsnorm_quant(h, ht, m, k, gamma_folded[c], eps, act_scale[c], xq[c],
                                               c == 0 ? r_out : nullptr, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    NormConsumers cons{};
    for (int c = 0; c < n; ++c) {
        cons.gamma[c] = gamma_folded[c];
        cons.act_scale[c] = act_scale[c];
        cons.xq[c] = xq[c];
    }
    return ht == kBF16 ? launch_multi_n<2>(n, h, m, k, eps, cons, r_out, stream)
                       : launch_multi_n<4>(n, h, m, k, eps, cons, r_out, stream);
}

hipError_t fold_norm_weight(const float* gamma, const float* inv_s, int64_t k, float* out, hipStream_t stream) {
    fold_kernel<<<dim3((unsigned)((k + 255) / 256)), dim3(256), 0, stream>>>(gamma, inv_s, k, out);
    return hipGetLastError();
}

}  // namespace sqk
