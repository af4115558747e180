// norm.hip -- RMSNorm in front of a smoothed projection, with 1/s folded into
// the norm weight so the norm's output is already X/s and goes straight into
// the per-tensor quantizer (kwkr.cn blog §2.3 and §3.2: the per-channel 1/s is
// absorbed by the gamma of the preceding norm, once, offline, and the scaling
// still happens before the rounding).
//
// One block of 256 threads per row. The row's sum of squares is taken in
// fp64 (squares of bf16 or fp32 values are exact in fp64, so only the order
// of the additions is free), reduced across the block, and
// r = fp32(1 / sqrt(sum / k + eps)) is evaluated in fp64 and rounded once.
// Rows of up to 256 * 8 16-byte vectors (16384 bf16 or 8192 fp32 values) stay
// in registers between the reduction and the output pass; longer rows are
// read a second time (from L2).
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
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const double d = (double)e[i];
        s += d * d;
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
        int q[E];
#pragma unroll
        for (int i = 0; i < E; ++i) q[i] = sqd::q8(__fmul_rn(y[i], inv_a));
        if constexpr (E == 8)
            *(sqd::u32x2*)((int8_t*)out + idx) = sqd::u32x2{sqd::pack4_i8(q[0], q[1], q[2], q[3]),
                                                             sqd::pack4_i8(q[4], q[5], q[6], q[7])};
        else
            *(uint32_t*)((int8_t*)out + idx) = sqd::pack4_i8(q[0], q[1], q[2], q[3]);
    }
}

// VPT > 0: the row is held in VPT vectors per thread (kvec <= 256 * VPT).
// VPT == 0: the row is streamed twice.
template <int EB, int VPT, NormOut OUT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const u32x4* __restrict__ h, int64_t kvec, int64_t k,
                                                               const float* __restrict__ gamma, float eps,
                                                               const float* __restrict__ act_scale,
                                                               void* __restrict__ out, float* __restrict__ r_out) {
    constexpr int E = 16 / EB;
    __shared__ double red[kNormWaves];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const u32x4* hr = h + row * kvec;

    double ss = 0.0;
    u32x4 v[VPT > 0 ? VPT : 1];
    if constexpr (VPT > 0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t c = tid + (int64_t)i * kNormThreads;
            v[i] = c < kvec ? __builtin_nontemporal_load(hr + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) ss += sum_sq<E>(v[i]);
    } else {
        for (int64_t c = tid; c < kvec; c += kNormThreads) ss += sum_sq<E>(hr[c]);
    }
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    double total = red[0];
#pragma unroll
    for (int w = 1; w < kNormWaves; ++w) total += red[w];
    const float r = (float)(1.0 / sqrt(total / (double)k + (double)eps));
    if (r_out && tid == 0) r_out[row] = r;
    const float inv_a = OUT == kOutI8 ? __fdiv_rn(1.0f, act_scale[0]) : 0.0f;

    if constexpr (VPT > 0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t c = tid + (int64_t)i * kNormThreads;
            if (c < kvec) {
                float g[E];
                load_gamma<E>(gamma, c, g);
                emit<E, OUT>(v[i], r, g, inv_a, out, row * k + c * E);
            }
        }
    } else {
        for (int64_t c = tid; c < kvec; c += kNormThreads) {
            float g[E];
            load_gamma<E>(gamma, c, g);
            emit<E, OUT>(hr[c], r, g, inv_a, out, row * k + c * E);
        }
    }
}

template <int EB, NormOut OUT>
hipError_t launch_norm(const void* h, int64_t m, int64_t k, const float* gamma, float eps, const float* act_scale,
                       void* out, float* r_out, hipStream_t stream) {
    const int64_t kvec = k * EB / 16;
    const dim3 grid((unsigned)m), block(kNormThreads);
    const u32x4* hp = (const u32x4*)h;
    if (kvec <= 1 * kNormThreads)
        rmsnorm_kernel<EB, 1, OUT><<<grid, block, 0, stream>>>(hp, kvec, k, gamma, eps, act_scale, out, r_out);
    else if (kvec <= 2 * kNormThreads)
        rmsnorm_kernel<EB, 2, OUT><<<grid, block, 0, stream>>>(hp, kvec, k, gamma, eps, act_scale, out, r_out);
    else if (kvec <= 4 * kNormThreads)
        rmsnorm_kernel<EB, 4, OUT><<<grid, block, 0, stream>>>(hp, kvec, k, gamma, eps, act_scale, out, r_out);
    else if (kvec <= 8 * kNormThreads)
        rmsnorm_kernel<EB, 8, OUT><<<grid, block, 0, stream>>>(hp, kvec, k, gamma, eps, act_scale, out, r_out);
    else
        rmsnorm_kernel<EB, 0, OUT><<<grid, block, 0, stream>>>(hp, kvec, k, gamma, eps, act_scale, out, r_out);
    return hipGetLastError();
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

hipError_t fold_norm_weight(const float* gamma, const float* inv_s, int64_t k, float* out, hipStream_t stream) {
    fold_kernel<<<dim3((unsigned)((k + 255) / 256)), dim3(256), 0, stream>>>(gamma, inv_s, k, out);
    return hipGetLastError();
}

}  // namespace sqk
