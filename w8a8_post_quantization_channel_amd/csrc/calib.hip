// calib.hip -- calibration statistics and smoothing factors.
//
// absmax: per-input-channel max |x| over the rows of a row-major [rows, k]
// matrix (the calibration statistic of the kwkr.cn blog §3.1, kept as a
// running max across batches like ADR-010's add_batch; the same reduction on
// W[n,k] gives max|W_j| over output rows).
//
// The reduction is done on magnitudes as integers: for finite IEEE values
// |x| ordered as a float equals (bits & ~sign) ordered as an unsigned integer,
// and bf16 bits widen to fp32 bits by a 16-bit shift, so the maximum is exact
// and needs no float compare. Each wave reads one row segment of 64 x 16 B
// (fully coalesced); the four waves of a block take interleaved rows and
// combine through LDS; one atomicMax per column per block merges blocks.
#include <algorithm>

#include <mutex>

#include "sq_device.h"
#include "sq_kernels.h"

namespace {

using sqd::item_of;
using sqd::u32x4;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kAbsThreads = 256;  // 4 waves
constexpr int kAbsUnroll = 8;     // 16-byte loads in flight per lane
constexpr int kAbsMinRows = 32;   // rows per block (at least): bounds the per-block atomics

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    u16x2 va = __builtin_bit_cast(u16x2, a), vb = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(va, vb));
}

// per-word running maximum of magnitudes for one 16-byte vector
template <int EB>
__device__ __forceinline__ void acc_mag(u32x4& m, const u32x4& v) {
    if constexpr (EB == 2) {
        m.x = max_u16x2(m.x, v.x & 0x7fff7fffu);
        m.y = max_u16x2(m.y, v.y & 0x7fff7fffu);
        m.z = max_u16x2(m.z, v.z & 0x7fff7fffu);
        m.w = max_u16x2(m.w, v.w & 0x7fff7fffu);
    } else {
        m.x = max(m.x, v.x & 0x7fffffffu);
        m.y = max(m.y, v.y & 0x7fffffffu);
        m.z = max(m.z, v.z & 0x7fffffffu);
        m.w = max(m.w, v.w & 0x7fffffffu);
    }
}

// fp32 bit pattern of the magnitude of column c of a strip, taken from the
// per-lane word vector `w` of the lane that loaded it
template <int EB>
__device__ __forceinline__ uint32_t column_bits(const uint32_t* words, int c) {
    if constexpr (EB == 2) {
        const uint32_t wd = words[(c >> 1) & 3];
        return (c & 1) ? (wd & 0xffff0000u) : (wd << 16);
    } else {
        return words[c & 3];
    }
}

// Block = 4 waves over one strip of 64 16-byte column vectors and a chunk of
// rows; wave w takes rows r0 + w, r0 + w + 4, ... with kAbsUnroll loads in
// flight per lane. The four wave partials meet in LDS; then every thread
// merges whole columns so each atomic instruction covers consecutive
// addresses. kPerChunk: each row chunk is one calibration sample and its
// maxima are stored to row `chunk` of out (no atomics, no zero fill).
template <int EB, bool kPerChunk>
__device__ __forceinline__ void absmax_block(const u32x4* __restrict__ x, int64_t rows, int64_t kvec, int64_t k,
                                             int64_t rows_per_block, unsigned* __restrict__ out_bits,
                                             int64_t strip, int64_t chunk, u32x4* part) {
    constexpr int E = 16 / EB;          // elements per 16-byte vector
    constexpr int COLS = 64 * E;        // columns per strip
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t v = strip * 64 + lane;  // 16-byte column vector
    const int64_t r0 = chunk * rows_per_block;
    const int64_t r1 = min(rows, r0 + rows_per_block);
    u32x4 m = u32x4{0u, 0u, 0u, 0u};
    if (v < kvec) {
        int64_t r = r0 + wave;
        const u32x4* p = x + r * kvec + v;
        const int64_t step = 4 * kvec;
        for (; r + 4 * (kAbsUnroll - 1) < r1; r += 4 * kAbsUnroll) {
            u32x4 t[kAbsUnroll];
#pragma unroll
            for (int u = 0; u < kAbsUnroll; ++u) t[u] = __builtin_nontemporal_load(p + u * step);
#pragma unroll
            for (int u = 0; u < kAbsUnroll; ++u) acc_mag<EB>(m, t[u]);
            p += kAbsUnroll * step;
        }
        for (; r < r1; r += 4) {
            acc_mag<EB>(m, __builtin_nontemporal_load(p));
            p += step;
        }
    }
    part[threadIdx.x] = m;
    __syncthreads();
    const int64_t col0 = strip * COLS;
#pragma unroll
    for (int c = threadIdx.x; c < COLS; c += kAbsThreads) {
        if (col0 + c >= k) break;
        uint32_t best = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const u32x4 pv = part[w * 64 + c / E];
            const uint32_t words[4] = {pv.x, pv.y, pv.z, pv.w};
            best = max(best, column_bits<EB>(words, c));
        }
        if constexpr (kPerChunk)
            out_bits[chunk * k + col0 + c] = best;
        else
            atomicMax(out_bits + col0 + c, best);
    }
}

// per-sample maxima: grid (strips, samples)
template <int EB>
__global__ __launch_bounds__(kAbsThreads) void sample_max_kernel(const u32x4* __restrict__ x, int64_t rows,
                                                                 int64_t kvec, int64_t k, int64_t rows_per_sample,
                                                                 unsigned* __restrict__ out_bits) {
    __shared__ u32x4 part[kAbsThreads];
    absmax_block<EB, true>(x, rows, kvec, k, rows_per_sample, out_bits, blockIdx.x, blockIdx.y, part);
}

// Several inputs in one launch (the projections of a block): item i owns the
// blocks [first[i], first[i + 1]) of a 1-D grid, laid out strip-fastest as a
// (strips, chunks) grid of its own would be. The item is uniform per block.
struct AbsTable {
    int count;
    int32_t first[sqk::kMaxBatch + 1];
    const u32x4* x[sqk::kMaxBatch];
    unsigned* out[sqk::kMaxBatch];
    int64_t rows[sqk::kMaxBatch], kvec[sqk::kMaxBatch], k[sqk::kMaxBatch], rpb[sqk::kMaxBatch];
    int32_t strips[sqk::kMaxBatch], eb[sqk::kMaxBatch];
};

__global__ __launch_bounds__(kAbsThreads) void absmax_batched_kernel(const AbsTable tab) {
    __shared__ u32x4 part[kAbsThreads];
    const int32_t b = blockIdx.x;
    const int i = item_of(tab.first, tab.count, b);
    const int32_t local = b - tab.first[i];
    // integer division has no scalar instruction: bring the block-uniform
    // quotient back to a scalar register so everything derived from it is too
    const int32_t chunk = __builtin_amdgcn_readfirstlane(local / tab.strips[i]), strip = local - chunk * tab.strips[i];
    if (tab.eb[i] == 2)
        absmax_block<2, false>(tab.x[i], tab.rows[i], tab.kvec[i], tab.k[i], tab.rpb[i], tab.out[i], strip, chunk,
                               part);
    else
        absmax_block<4, false>(tab.x[i], tab.rows[i], tab.kvec[i], tab.k[i], tab.rpb[i], tab.out[i], strip, chunk,
                               part);
}

// zeros over several buffers in one launch: buffer i owns blocks
// [first[i], first[i + 1]) of 256 floats each
struct FillTable {
    int count;
    int32_t first[sqk::kMaxBatch + 1];
    float* p[sqk::kMaxBatch];
    int64_t n[sqk::kMaxBatch];
};

__global__ __launch_bounds__(256) void fill_zero_batched_kernel(const FillTable tab) {
    const int i = item_of(tab.first, tab.count, blockIdx.x);
    const int64_t j = (int64_t)(blockIdx.x - tab.first[i]) * 256 + threadIdx.x;
    if (j < tab.n[i]) tab.p[i][j] = 0.0f;
}

// Running fp64 sum of per-sample maxima, one thread per channel, the samples
// added strictly in order (so the result does not depend on the launch
// shape); kSumBatch loads are issued before their additions.
constexpr int kSumThreads = 256;
constexpr int kSumBatch = 16;

__global__ __launch_bounds__(kSumThreads) void sum_samples_kernel(const float* __restrict__ sample_max,
                                                                  int64_t samples, int64_t k,
                                                                  double* __restrict__ sum) {
    const int64_t j = (int64_t)blockIdx.x * kSumThreads + threadIdx.x;
    if (j >= k) return;
    double acc = sum[j];
    int64_t b = 0;
    for (; b + kSumBatch <= samples; b += kSumBatch) {
        float v[kSumBatch];
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) v[u] = sample_max[(b + u) * k + j];
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) acc += (double)v[u];
    }
    for (; b < samples; ++b) acc += (double)sample_max[b * k + j];
    sum[j] = acc;
}

__global__ __launch_bounds__(kSumThreads) void mean_finalize_kernel(const double* __restrict__ sum, double count,
                                                                    int64_t k, float* __restrict__ act_max) {
    const int64_t j = (int64_t)blockIdx.x * kSumThreads + threadIdx.x;
    if (j < k) act_max[j] = (float)(sum[j] / count);
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// s_j = max|X_j|^alpha / max|W_j|^(1-alpha) (kwkr.cn blog §2.2): fp64 pow and
// quotient, one rounding to fp32; inv_s_j = fp32(1/s_j). One thread per channel.
constexpr int kSmoothThreads = 256;

// H: s is stored as binary16 (ADR-010 "Consequences") and inv_s is not
// written: its users form fl(1 / decoded s) themselves.
template <bool H>
__device__ __forceinline__ void smooth_channel(const float* __restrict__ act_max, const float* __restrict__ w_max,
                                               int64_t j, double alpha, void* __restrict__ s,
                                               float* __restrict__ inv_s) {
    const float a = __builtin_fmaxf(act_max[j], sqd::kFloor);
    const float w = __builtin_fmaxf(w_max[j], sqd::kFloor);
    const double num = pow((double)a, alpha);
    const double den = pow((double)w, 1.0 - alpha);
    const float sj = (float)(num / den);
    if constexpr (H) {
        ((uint16_t*)s)[j] = sqd::scale_f16(sj);
    } else {
        ((float*)s)[j] = sj;
        inv_s[j] = __fdiv_rn(1.0f, sj);
    }
}

// Closed-form per-tensor activation scale (ADR-010 "Key design" item 1):
// act_scale = fp32( max_j fp32(max(act_max[j], 1e-5) * inv_s[j]) / 127 ).
constexpr int kScaleThreads = 1024;

// H: the factors are the stored binary16 s (inv = fl(1 / decoded s)) and the
// scale is stored as binary16.
template <bool H>
__device__ __forceinline__ float inv_at(const void* __restrict__ inv_s, int64_t j) {
    if constexpr (H)
        return sqd::f16_inv(((const uint16_t*)inv_s)[j]);
    else
        return ((const float*)inv_s)[j];
}

template <bool H>
__device__ __forceinline__ void act_scale_block(const float* __restrict__ act_max, const void* __restrict__ inv_s,
                                                int64_t k, float qmax, void* __restrict__ act_scale, float* red) {
    // four channels per thread per round, their eight loads issued together
    // (the max is exact, so the order does not change the result)
    float mx = 0.0f;
    int64_t j = threadIdx.x;
    for (; j + 3 * kScaleThreads < k; j += 4 * kScaleThreads) {
        float a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = act_max[j + u * kScaleThreads];
            b[u] = inv_at<H>(inv_s, j + u * kScaleThreads);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) mx = __builtin_fmaxf(mx, __fmul_rn(__builtin_fmaxf(a[u], sqd::kFloor), b[u]));
    }
    for (; j < k; j += kScaleThreads)
        mx = __builtin_fmaxf(mx, __fmul_rn(__builtin_fmaxf(act_max[j], sqd::kFloor), inv_at<H>(inv_s, j)));
    mx = sqd::block_max<kScaleThreads / 64>(mx, red);
    if (threadIdx.x == 0) {
        const float sc = __fdiv_rn(mx, qmax);
        if constexpr (H)
            ((uint16_t*)act_scale)[0] = sqd::scale_f16(sc);
        else
            ((float*)act_scale)[0] = sc;
    }
}

__global__ __launch_bounds__(kScaleThreads) void act_scale_kernel(const float* __restrict__ act_max,
                                                                  const float* __restrict__ inv_s, int64_t k,
                                                                  float qmax, float* __restrict__ act_scale) {
    __shared__ float red[kScaleThreads / 64];
    act_scale_block<false>(act_max, inv_s, k, qmax, act_scale, red);
}

// Smoothing factors of several projections: item i owns blocks
// [first[i], first[i + 1]) of the smoothing launch and block i of the scale
// launch.
struct SmoothTable {
    int count;
    int32_t first[sqk::kMaxBatch + 1];
    const float* act_max[sqk::kMaxBatch];
    const float* w_max[sqk::kMaxBatch];
    int64_t k[sqk::kMaxBatch];
    double alpha[sqk::kMaxBatch];
    void* s[sqk::kMaxBatch];
    float* inv_s[sqk::kMaxBatch];
    void* act_scale[sqk::kMaxBatch];
};

template <bool H>
__global__ __launch_bounds__(kSmoothThreads) void smooth_batched_kernel(const SmoothTable tab) {
    const int i = item_of(tab.first, tab.count, blockIdx.x);
    const int64_t j = (int64_t)(blockIdx.x - tab.first[i]) * kSmoothThreads + threadIdx.x;
    if (j < tab.k[i]) smooth_channel<H>(tab.act_max[i], tab.w_max[i], j, tab.alpha[i], tab.s[i], tab.inv_s[i]);
}

// qmax: 127 for int8 codes, 448 for e4m3 codes; H: the factors are read from
// the stored binary16 s
template <bool H>
__global__ __launch_bounds__(kScaleThreads) void act_scale_batched_kernel(const SmoothTable tab, float qmax) {
    __shared__ float red[kScaleThreads / 64];
    const int i = blockIdx.x;
    act_scale_block<H>(tab.act_max[i], H ? tab.s[i] : tab.inv_s[i], tab.k[i], qmax, tab.act_scale[i], red);
}

// launch geometry of one absmax input: about 2048 blocks, but at least
// kAbsMinRows rows per block (fewer atomics), rows per block a multiple of
// 4 waves x kAbsUnroll
struct AbsGeom {
    int64_t kvec, strips, rpb, chunks;
};

// Rows of 64-vector column strips a launch reads (rows x strips summed over
// its inputs). Every block ends with one device-scope atomicMax per column,
// and those go past the (per-XCD) L2 to memory: a launch with at least
// kAbsBigWork of them takes about 256 blocks per input and at least 256 rows
// per block (measured on MI355X: the 13B block's eleven statistics 124 ->
// 116 us, a 262144 x 5120 calibration tensor 6.8 -> 7.06 TB/s; 7.4 M -> 1.0 M
// atomics per 13B step); smaller launches keep more, shorter blocks so a
// single small input still fills the compute units.
constexpr int64_t kAbsBigWork = 262144;

AbsGeom abs_geom(int eb, int64_t rows, int64_t k, bool big) {
    AbsGeom g;
    g.kvec = k * eb / 16;
    g.strips = (g.kvec + 63) / 64;
    const int64_t granule = 4 * kAbsUnroll;
    const int64_t target_chunks = std::max<int64_t>(1, (big ? 256 : 2048) / g.strips);
    int64_t rpb = (rows + target_chunks - 1) / target_chunks;
    rpb = std::max<int64_t>(rpb, std::min<int64_t>(rows, big ? 8 * kAbsMinRows : kAbsMinRows));
    g.rpb = std::max<int64_t>(granule, (rpb + granule - 1) / granule * granule);
    g.chunks = (rows + g.rpb - 1) / g.rpb;
    return g;
}

}  // namespace

namespace sqk {

hipError_t absmax_batched(const AbsmaxItem* items, int count, bool accumulate, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    if (!accumulate) {
        FillTable ft{};
        ft.count = count;
        int64_t blocks = 0;
        for (int i = 0; i < count; ++i) {
            ft.first[i] = (int32_t)blocks;
            ft.p[i] = items[i].absmax;
            ft.n[i] = items[i].k;
            blocks += (items[i].k + 255) / 256;
        }
        if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        ft.first[count] = (int32_t)blocks;
        fill_zero_batched_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(ft);
    }
    int64_t work = 0;  // row-strips of the launch
    for (int i = 0; i < count; ++i)
        work += items[i].rows * ((items[i].k * elem_bytes(items[i].xt) / 16 + 63) / 64);
    const bool big = work >= kAbsBigWork;
    AbsTable tab{};
    int n = 0;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        if (items[i].rows == 0) continue;
        const int eb = elem_bytes(items[i].xt);
        const AbsGeom g = abs_geom(eb, items[i].rows, items[i].k, big);
        tab.first[n] = (int32_t)blocks;
        tab.x[n] = (const u32x4*)items[i].x;
        tab.out[n] = (unsigned*)items[i].absmax;
        tab.rows[n] = items[i].rows;
        tab.kvec[n] = g.kvec;
        tab.k[n] = items[i].k;
        tab.rpb[n] = g.rpb;
        tab.strips[n] = (int32_t)g.strips;
        tab.eb[n] = eb;
        blocks += g.strips * g.chunks;
        ++n;
    }
    if (n == 0) return hipGetLastError();
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    tab.count = n;
    tab.first[n] = (int32_t)blocks;
    absmax_batched_kernel<<<dim3((unsigned)blocks), dim3(kAbsThreads), 0, stream>>>(tab);
    return hipGetLastError();
}

hipError_t absmax(const void* x, int xt, int64_t rows, int64_t k, float* absmax_out, bool accumulate,
                  hipStream_t stream) {
    const AbsmaxItem item{x, xt, rows, k, absmax_out};
    return absmax_batched(&item, 1, accumulate, stream);
}

hipError_t act_scale(const float* act_max, const float* inv_s, int64_t k, float* act_scale_out,
                     hipStream_t stream) {
    act_scale_kernel<<<dim3(1), dim3(kScaleThreads), 0, stream>>>(act_max, inv_s, k, sqd::kQmax, act_scale_out);
    return hipGetLastError();
}

hipError_t act_scale_fp8(const float* act_max, const float* inv_s, int64_t k, float* act_scale_out,
                         hipStream_t stream) {
    act_scale_kernel<<<dim3(1), dim3(kScaleThreads), 0, stream>>>(act_max, inv_s, k, sqd::kFp8Max, act_scale_out);
    return hipGetLastError();
}

hipError_t sample_max(const void* x, int xt, int64_t samples, int64_t rows_per_sample, int64_t k,
                      float* sample_max_out, hipStream_t stream) {
    const int eb = elem_bytes(xt);
    const int64_t kvec = k * eb / 16;
    const int64_t strips = (kvec + 63) / 64;
    const int64_t rows = samples * rows_per_sample;
    // one block per (column strip, sample); samples beyond the 65535 grid
    // rows are taken by further launches
    for (int64_t b0 = 0; b0 < samples; b0 += 65535) {
        const int64_t nb = std::min<int64_t>(65535, samples - b0);
        const dim3 grid((unsigned)strips, (unsigned)nb);
        const int64_t off = b0 * rows_per_sample * kvec;
        unsigned* out = (unsigned*)(sample_max_out + b0 * k);
        const int64_t r = std::min<int64_t>(rows - b0 * rows_per_sample, nb * rows_per_sample);
        if (eb == 2)
            sample_max_kernel<2><<<grid, dim3(kAbsThreads), 0, stream>>>((const u32x4*)x + off, r, kvec, k,
                                                                          rows_per_sample, out);
        else
            sample_max_kernel<4><<<grid, dim3(kAbsThreads), 0, stream>>>((const u32x4*)x + off, r, kvec, k,
                                                                          rows_per_sample, out);
    }
    return hipGetLastError();
}

hipError_t sum_samples(const float* sample_max_in, int64_t samples, int64_t k, double* sum, hipStream_t stream) {
    sum_samples_kernel<<<dim3((unsigned)((k + kSumThreads - 1) / kSumThreads)), dim3(kSumThreads), 0, stream>>>(
        sample_max_in, samples, k, sum);
    return hipGetLastError();
}

hipError_t mean_finalize(const double* sum, int64_t count, int64_t k, float* act_max, hipStream_t stream) {
    mean_finalize_kernel<<<dim3((unsigned)((k + kSumThreads - 1) / kSumThreads)), dim3(kSumThreads), 0,
                           stream>>>(sum, (double)count, k, act_max);
    return hipGetLastError();
}

// every item of one call has the same storage (items[0].h)
static hipError_t smooth_factors_batched_q(const SmoothItem* items, int count, float qmax, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const bool h = items[0].h;
    for (int i = 1; i < count; ++i)
        if (items[i].h != h) return hipErrorInvalidValue;
    SmoothTable tab{};
    tab.count = count;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        tab.first[i] = (int32_t)blocks;
        tab.act_max[i] = items[i].act_max;
        tab.w_max[i] = items[i].w_max;
        tab.k[i] = items[i].k;
        tab.alpha[i] = (double)items[i].alpha;
        tab.s[i] = items[i].s;
        tab.inv_s[i] = items[i].inv_s;
        tab.act_scale[i] = items[i].act_scale;
        blocks += (items[i].k + kSmoothThreads - 1) / kSmoothThreads;
    }
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    tab.first[count] = (int32_t)blocks;
    if (h) {
        smooth_batched_kernel<true><<<dim3((unsigned)blocks), dim3(kSmoothThreads), 0, stream>>>(tab);
        act_scale_batched_kernel<true><<<dim3((unsigned)count), dim3(kScaleThreads), 0, stream>>>(tab, qmax);
    } else {
        smooth_batched_kernel<false><<<dim3((unsigned)blocks), dim3(kSmoothThreads), 0, stream>>>(tab);
        act_scale_batched_kernel<false><<<dim3((unsigned)count), dim3(kScaleThreads), 0, stream>>>(tab, qmax);
    }
    return hipGetLastError();
}

hipError_t smooth_factors_batched(const SmoothItem* items, int count, hipStream_t stream) {
    return smooth_factors_batched_q(items, count, sqd::kQmax, stream);
}

hipError_t act_scale_batched(const SmoothItem* items, int count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    SmoothTable tab{};
    tab.count = count;
    for (int i = 0; i < count; ++i) {
        tab.act_max[i] = items[i].act_max;
        tab.inv_s[i] = items[i].inv_s;
        tab.k[i] = items[i].k;
        tab.act_scale[i] = items[i].act_scale;
    }
    act_scale_batched_kernel<false><<<dim3((unsigned)count), dim3(kScaleThreads), 0, stream>>>(tab, sqd::kQmax);
    return hipGetLastError();
}

hipError_t smooth_factors_fp8_batched(const SmoothItem* items, int count, hipStream_t stream) {
    return smooth_factors_batched_q(items, count, sqd::kFp8Max, stream);
}

hipError_t smooth_factors(const float* act_max, const float* w_max, int64_t k, float alpha, float* s,
                          float* inv_s, float* act_scale, hipStream_t stream) {
    const SmoothItem item{act_max, w_max, k, alpha, s, inv_s, act_scale, false};
    return smooth_factors_batched(&item, 1, stream);
}

}  // namespace sqk

// ---- nearest-rank percentile of |x| per channel (kwkr.cn blog §3.1) -----------
//
// Radix selection on the magnitude bit patterns (finite IEEE values order like
// their bits with the sign cleared): 15-bit keys for bf16, 31-bit for fp32,
// taken 8 bits at a time from the top (bf16: 8 + 7, fp32: 8 + 8 + 8 + 7). A
// pass histograms the next digit of every key whose higher digits equal the
// prefix selected so far, then one thread per channel walks its histogram to
// the bucket holding the remaining rank. All counts are integers, so the
// result is exact and independent of the launch shape.
namespace {

constexpr int kPctThreads = 1024;  // 16 waves over interleaved rows
constexpr int kPctChannels = 64;   // one channel per lane
constexpr int kPctBins = 256;
constexpr int kPctRows = kPctBins;        // LDS histogram rows, one per bin
constexpr int kPctUnroll = 16;

template <int EB>
struct PctKey {
    static constexpr int BITS = EB == 2 ? 15 : 31;
    static constexpr int PASSES = (BITS + 7) / 8;
    // bit position of the lowest bit of digit `pass` and its width
    __host__ __device__ static constexpr int lo(int pass) { return BITS - 8 * (pass + 1) > 0 ? BITS - 8 * (pass + 1) : 0; }
    __host__ __device__ static constexpr int width(int pass) { return (BITS - 8 * pass) - lo(pass); }
};

template <int EB>
__device__ __forceinline__ uint32_t mag_key(const void* x, int64_t idx) {
    if constexpr (EB == 2)
        return (uint32_t)__builtin_nontemporal_load((const uint16_t*)x + idx) & 0x7fffu;
    else
        return __builtin_nontemporal_load((const uint32_t*)x + idx) & 0x7fffffffu;
}

template <int EB, int PASS>
__global__ __launch_bounds__(kPctThreads) void pct_hist_kernel(const void* __restrict__ x, int64_t rows, int64_t k,
                                                               int64_t rows_per_block,
                                                               const uint32_t* __restrict__ prefix,
                                                               uint32_t* __restrict__ hist) {
    using K = PctKey<EB>;
    constexpr int LO = K::lo(PASS), HI = LO + K::width(PASS);
    constexpr uint32_t DMASK = (1u << K::width(PASS)) - 1u;
    // bin-major: lane l's bin d is word d * 64 + l, in bank l whatever the
    // digits, so the 64 lanes of an atomic never share a bank (a lane-major
    // row per channel puts bin d in bank (l + d) % 64, and digits that differ
    // across lanes, like the low digit of the later passes, then collide)
    __shared__ uint32_t h[kPctRows * kPctChannels];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kPctRows * kPctChannels; i += kPctThreads) h[i] = 0u;
    __syncthreads();
    const int64_t c = (int64_t)blockIdx.x * kPctChannels + lane;  // k is a multiple of 64
    const uint32_t pre = PASS > 0 ? prefix[c] : 0u;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = min(rows, r0 + rows_per_block);
    constexpr int W = kPctThreads / 64;
    // keys outside the selected prefix are skipped (their lanes sit the
    // atomic out): at a high percentile almost every key of the later passes
    // is outside, and counting them all in one pad word chained 16
    // read-modify-writes per lane on one address
    auto count = [&](uint32_t key) {
        if (PASS == 0 || (key >> HI) == pre) atomicAdd(&h[((key >> LO) & DMASK) * kPctChannels + lane], 1u);
    };
    int64_t r = r0 + wave;
    for (; r + W * (kPctUnroll - 1) < r1; r += W * kPctUnroll) {
        uint32_t key[kPctUnroll];
#pragma unroll
        for (int u = 0; u < kPctUnroll; ++u) key[u] = mag_key<EB>(x, (r + W * u) * k + c);
#pragma unroll
        for (int u = 0; u < kPctUnroll; ++u) count(key[u]);
    }
    for (; r < r1; r += W) count(mag_key<EB>(x, r * k + c));
    __syncthreads();
    // merge: lane l takes channel l (bank l again) and each wave 16
    // consecutive bins
    const int ch = lane, b0 = wave * 16;
    uint32_t* g = hist + ((int64_t)blockIdx.x * kPctChannels + ch) * kPctBins;
#pragma unroll
    for (int b = b0; b < b0 + 16; ++b) {
        const uint32_t v = h[b * kPctChannels + ch];
        if (v) atomicAdd(g + b, v);
    }
}

// One thread per channel: the bucket of this pass's digit that holds the
// remaining rank (1-based, counted from the smallest key).
template <int EB, int PASS>
__global__ __launch_bounds__(256) void pct_select_kernel(const uint32_t* __restrict__ hist, int64_t k,
                                                         uint32_t rank0, uint32_t* __restrict__ prefix,
                                                         uint32_t* __restrict__ rank, float* __restrict__ act_max) {
    using K = PctKey<EB>;
    constexpr int NB = 1 << K::width(PASS);
    constexpr bool LAST = PASS == K::PASSES - 1;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= k) return;
    uint32_t r = PASS == 0 ? rank0 : rank[c];
    const uint32_t* hc = hist + c * kPctBins;
    uint32_t cum = 0;
    int d = 0;
    for (; d < NB - 1; ++d) {
        const uint32_t n = hc[d];
        if (cum + n >= r) break;
        cum += n;
    }
    r -= cum;
    const uint32_t pre = ((PASS == 0 ? 0u : prefix[c]) << K::width(PASS)) | (uint32_t)d;
    if constexpr (LAST) {
        act_max[c] = __uint_as_float(EB == 2 ? pre << 16 : pre);
    } else {
        prefix[c] = pre;
        rank[c] = r;
    }
}

__global__ __launch_bounds__(256) void fill_zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <int EB, int PASS>
hipError_t pct_pass(const void* x, int64_t rows, int64_t k, uint32_t rank0, uint32_t* hist, uint32_t* prefix,
                    uint32_t* rank, float* act_max, hipStream_t stream) {
    const int64_t strips = k / kPctChannels;
    // about ten blocks per compute unit, at least 1024 rows per block
    int64_t chunks = std::max<int64_t>(1, 2560 / strips);
    int64_t rpb = std::max<int64_t>(1024, (rows + chunks - 1) / chunks);
    chunks = std::min<int64_t>(65535, (rows + rpb - 1) / rpb);
    rpb = (rows + chunks - 1) / chunks;
    uint32_t* hp = hist + (int64_t)PASS * k * kPctBins;
    pct_hist_kernel<EB, PASS><<<dim3((unsigned)strips, (unsigned)chunks), dim3(kPctThreads), 0, stream>>>(
        x, rows, k, rpb, prefix, hp);
    pct_select_kernel<EB, PASS><<<dim3((unsigned)((k + 255) / 256)), dim3(256), 0, stream>>>(hp, k, rank0, prefix,
                                                                                          rank, act_max);
    return hipGetLastError();
}

template <int EB>
hipError_t percentile_t(const void* x, int64_t rows, int64_t k, uint32_t rank0, uint32_t* hist, uint32_t* prefix,
                        uint32_t* rank, float* act_max, hipStream_t stream) {
    const int64_t words = (int64_t)PctKey<EB>::PASSES * k * kPctBins;
    fill_zero_u32_kernel<<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream>>>(hist, words);
    hipError_t e = pct_pass<EB, 0>(x, rows, k, rank0, hist, prefix, rank, act_max, stream);
    if (e == hipSuccess) e = pct_pass<EB, 1>(x, rows, k, rank0, hist, prefix, rank, act_max, stream);
    if constexpr (PctKey<EB>::PASSES > 2) {
        if (e == hipSuccess) e = pct_pass<EB, 2>(x, rows, k, rank0, hist, prefix, rank, act_max, stream);
        if (e == hipSuccess) e = pct_pass<EB, 3>(x, rows, k, rank0, hist, prefix, rank, act_max, stream);
    }
    return e;
}

}  // namespace

// ---- the percentile's scratch without allocation ----------------------------------
//
// For callers that cannot allocate, the histograms, prefixes and ranks live
// in one file-scope device array. Its host-side name is a stand-in, not a
// device address: every use goes through the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
namespace {

constexpr size_t kPctScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint32_t scratch[kPctScratchBytes / 4];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace sqk {

size_t percentile_scratch_bytes() { return kPctScratchBytes; }

hipError_t percentile_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t percentile_workspace(int xt, int64_t k) {
    const int passes = xt == kBF16 ? PctKey<2>::PASSES : PctKey<4>::PASSES;
    return (size_t)passes * (size_t)k * kPctBins * 4 + 2 * (size_t)k * 4;
}

hipError_t percentile(const void* x, int xt, int64_t rows, int64_t k, int64_t rank, void* workspace,
                      float* act_max, hipStream_t stream) {
    const int passes = xt == kBF16 ? PctKey<2>::PASSES : PctKey<4>::PASSES;
    uint32_t* hist = (uint32_t*)workspace;
    uint32_t* prefix = hist + (int64_t)passes * k * kPctBins;
    uint32_t* rnk = prefix + k;
    if (xt == kBF16) return percentile_t<2>(x, rows, k, (uint32_t)rank, hist, prefix, rnk, act_max, stream);
    return percentile_t<4>(x, rows, k, (uint32_t)rank, hist, prefix, rnk, act_max, stream);
}

}  // namespace sqk
