// gemm.hip -- the INT8 x INT8 -> INT32 product of the W8A8 layer on CDNA4
// matrix cores, with the dequantization fused into the epilogue (the scale
// multiplications merged, as the pwwt.cn §3.1 kernel stub describes; the
// stub's tensor-core mma tiling is prior art for other hardware and is not
// followed here).
//
// Design (gfx950):
//   * v_mfma_i32_32x32x32_i8: each lane feeds 16 bytes of A (row lane%32) and
//     16 bytes of B (column lane%32) per instruction; A and B use the same
//     lane -> k-slot mapping, so the dot product is exact whatever order the
//     hardware sums k in. The bf16 reference product (alpha search) reuses the
//     whole pipeline with v_mfma_f32_32x32x16_bf16, which has the same
//     16-bytes-per-lane operand shape.
//   * Block tile BM x BN over a BK = 128-byte K slab, two LDS stages. Global
//     loads are 16-byte chunks, 8 per 128-byte row segment; they are staged in
//     registers while the matrix cores work on the other LDS stage, so one
//     barrier per K slab suffices.
//   * LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
//     (row & 7): the 8 lanes that read one LDS phase hit 8 different bank
//     groups, both on the MFMA-fragment reads and on the staging writes.
//   * Tails: rows beyond M or N and K bytes beyond k are zero-filled in LDS,
//     which adds exact zeros to the integer sums.
//   * The tile index is remapped so consecutive tiles of one XCD share an A
//     row panel (workgroups are dealt round-robin over the 8 XCDs).
#include <algorithm>

#include "sq_device.h"
#include "sq_kernels.h"

namespace {

using sqd::u32x4;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct OpI8 {
    using acc_t = v16i;
    static constexpr int kElemBytes = 1;
    __device__ static __forceinline__ acc_t mfma(const v4i& a, const v4i& b, const acc_t& c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};

struct OpBF16 {
    using acc_t = v16f;
    static constexpr int kElemBytes = 2;
    __device__ static __forceinline__ acc_t mfma(const v4i& a, const v4i& b, const acc_t& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                       c, 0, 0, 0);
    }
};

constexpr int kBK = 128;  // bytes of K per LDS stage

// ---- epilogues ------------------------------------------------------------
// Each epilogue sees one 32x32 accumulator tile per call: lane owns column
// col and the 16 rows row_of(v); element v of `acc`.

// y = fp32(fp32(acc) * fp32(act_scale * w_scale[col])), fp32 or bf16 store;
// the raw int32 accumulator is stored too when acc_out is set.
template <bool kBF16Out>
struct EpiDequant {
    const float* act_scale;
    const float* w_scale;
    void* y;
    int32_t* acc_out;
    int64_t M, N;
    float a;
    __device__ void begin() { a = act_scale[0]; }
    template <class Acc>
    __device__ void tile(const Acc& acc, int64_t row0, int64_t col) {
        if (col >= N) return;
        const float c = __fmul_rn(a, w_scale[col]);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = row0 + 8 * (v >> 2) + (v & 3);
            if (row < M) {
                const int64_t idx = row * N + col;
                const float val = __fmul_rn((float)acc[v], c);
                if constexpr (kBF16Out)
                    ((uint16_t*)y)[idx] = (uint16_t)sqd::f32_to_bf16_bits(val);
                else
                    ((float*)y)[idx] = val;
                if (acc_out) acc_out[idx] = acc[v];
            }
        }
    }
    __device__ void end(char*) {}
};

// Squared error of the fp32 dequantized output against a reference, summed in
// fp64 per block into slots[blockIdx.x] (fixed-order tree, deterministic).
struct EpiSSE {
    const float* act_scale;
    const float* w_scale;
    const float* yref;
    double* slots;
    int64_t M, N;
    float a;
    double sum;
    __device__ void begin() {
        a = act_scale[0];
        sum = 0.0;
    }
    template <class Acc>
    __device__ void tile(const Acc& acc, int64_t row0, int64_t col) {
        if (col >= N) return;
        const float c = __fmul_rn(a, w_scale[col]);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = row0 + 8 * (v >> 2) + (v & 3);
            if (row < M) {
                const float val = __fmul_rn((float)acc[v], c);
                const double d = (double)val - (double)yref[row * N + col];
                sum += d * d;
            }
        }
    }
    __device__ void end(char* lds) {
        double* red = (double*)lds;
        red[threadIdx.x] = sum;
        __syncthreads();
        for (int w = blockDim.x / 2; w >= 1; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        if (threadIdx.x == 0) slots[blockIdx.x] = red[0];
    }
};

// plain fp32 store of the accumulator (reference product)
struct EpiStoreF32 {
    float* y;
    int64_t M, N;
    __device__ void begin() {}
    template <class Acc>
    __device__ void tile(const Acc& acc, int64_t row0, int64_t col) {
        if (col >= N) return;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = row0 + 8 * (v >> 2) + (v & 3);
            if (row < M) y[row * N + col] = (float)acc[v];
        }
    }
    __device__ void end(char*) {}
};

// ---- main kernel ------------------------------------------------------------

template <class Op, int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_kernel(const int8_t* __restrict__ A,
                                                                         const int8_t* __restrict__ B,
                                                                         int64_t M, int64_t N, int64_t Kb,
                                                                         int tiles_m, int tiles_n, Epi epi) {
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    constexpr int ROWS = BM + BN;
    constexpr int CPT = ROWS * (kBK / 16) / NT;  // 16-byte chunks per thread per stage
    static_assert(ROWS * (kBK / 16) % NT == 0, "stage must split evenly over threads");
    static_assert(NT % 8 == 0 && (NT / 8) * CPT == ROWS, "chunk rows must tile the stage");
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int STAGE = ROWS * kBK;
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous range of tiles (row-major over tiles_n) so tiles sharing an
    // A panel share that XCD's L2.
    const int ntiles = tiles_m * tiles_n;
    int t = blockIdx.x;
    {
        const int xcd = t & 7, slot = t >> 3;
        const int per = ntiles >> 3, rem = ntiles & 7;
        // XCD x owns tiles [x*per + min(x,rem), ...) of length per + (x < rem)
        t = xcd * per + min(xcd, rem) + slot;
    }
    const int tm = t / tiles_n, tn = t % tiles_n;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    // staging descriptors: chunk c of this thread covers row (tid/8 + c*NT/8)
    // of the stage, 16-byte column (tid % 8)
    const int kc = tid & 7;
    const int64_t kcb = kc * 16;
    const char* gsrc[CPT];
    bool ok[CPT];
    int ldst[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int row = (tid >> 3) + c * (NT / 8);
        int64_t grow;
        const int8_t* base;
        if (row < BM) {
            grow = m0 + row;
            ok[c] = grow < M;
            base = A;
        } else {
            grow = n0 + (row - BM);
            ok[c] = grow < N;
            base = B;
        }
        gsrc[c] = (const char*)base + (ok[c] ? grow * Kb : 0) + kcb;
        ldst[c] = row * kBK + ((kc ^ (row & 7)) << 4);
    }

    typename Op::acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = typename Op::acc_t{};

    u32x4 stg[CPT];
    auto gload = [&](int64_t kb) {
        const int64_t koff = kb * kBK;
        const bool kin = koff + kcb < Kb;
#pragma unroll
        for (int c = 0; c < CPT; ++c)
            stg[c] = (ok[c] && kin) ? *(const u32x4*)(gsrc[c] + koff) : u32x4{0u, 0u, 0u, 0u};
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) *(u32x4*)(lds + buf * STAGE + ldst[c]) = stg[c];
    };
    const int frag_row = lane & 31;
    auto compute = [&](int buf) {
        const char* sa = lds + buf * STAGE + (wm * WM + frag_row) * kBK;
        const char* sb = lds + buf * STAGE + (BM + wn * WN + frag_row) * kBK;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int chunk = ((2 * ks + (lane >> 5)) ^ (lane & 7)) << 4;
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const v4i*)(sa + i * 32 * kBK + chunk);
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = *(const v4i*)(sb + j * 32 * kBK + chunk);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Op::mfma(af[i], bf[j], acc[i][j]);
        }
    };

    const int64_t nk = (Kb + kBK - 1) / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int64_t kb = 0; kb < nk; ++kb) {
        const int cur = (int)(kb & 1);
        if (kb + 1 < nk) gload(kb + 1);
        compute(cur);
        if (kb + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    epi.begin();
    const int64_t rbase = m0 + wm * WM + 4 * (lane >> 5);
    const int64_t cbase = n0 + wn * WN + (lane & 31);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) epi.tile(acc[i][j], rbase + i * 32, cbase + j * 32);
    epi.end(lds);
}

// Tile configurations. Large: 256 x 256 block, 8 waves of 128 x 64.
// Small: 128 x 128 block, 4 waves of 64 x 64 (skinny M, small problems).
struct CfgLarge {
    static constexpr int BM = 256, BN = 256, WM = 128, WN = 64;
};
struct CfgSmall {
    static constexpr int BM = 128, BN = 128, WM = 64, WN = 64;
};

template <class Cfg>
constexpr int threads_of() {
    return (Cfg::BM / Cfg::WM) * (Cfg::BN / Cfg::WN) * 64;
}

template <class Op, class Cfg, class Epi>
hipError_t launch(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                  hipStream_t stream) {
    const int tiles_m = (int)((M + Cfg::BM - 1) / Cfg::BM);
    const int tiles_n = (int)((N + Cfg::BN - 1) / Cfg::BN);
    gemm_kernel<Op, Cfg::BM, Cfg::BN, Cfg::WM, Cfg::WN, Epi>
        <<<dim3((unsigned)(tiles_m * tiles_n)), dim3(threads_of<Cfg>()), 0, stream>>>(A, B, M, N, Kb, tiles_m,
                                                                                     tiles_n, epi);
    return hipGetLastError();
}

// Use the large tile when it still yields at least one tile per CU.
bool use_large(int64_t M, int64_t N) {
    const int64_t large_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    return M >= 256 && large_tiles >= 128;
}

__global__ __launch_bounds__(256) void reduce_slots_kernel(const double* __restrict__ slots, int64_t per_group,
                                                           double count, double* __restrict__ out) {
    __shared__ double red[256];
    const double* g = slots + (int64_t)blockIdx.x * per_group;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < per_group; i += 256) s += g[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] / count;
}

// fp32 reference product for fp32 inputs: 64x64 block tile, 4x4 per thread.
__global__ __launch_bounds__(256) void ref_gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                           int64_t M, int64_t N, int64_t K, float* __restrict__ Y) {
    __shared__ float xs[16][65];
    __shared__ float ws[16][65];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += 16) {
        for (int i = threadIdx.x; i < 64 * 16; i += 256) {
            const int r = i / 16, kk = i % 16;
            xs[kk][r] = (m0 + r < M) ? X[(m0 + r) * K + k0 + kk] : 0.0f;
            ws[kk][r] = (n0 + r < N) ? W[(n0 + r) * K + k0 + kk] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __fmaf_rn(xs[kk][ty * 4 + i], ws[kk][tx * 4 + j], acc[i][j]);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = m0 + ty * 4 + i, c = n0 + tx * 4 + j;
            if (r < M && c < N) Y[r * N + c] = acc[i][j];
        }
}

}  // namespace

namespace sqk {

hipError_t gemm_dequant(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                        const float* act_scale, const float* w_scale, void* y, int yt, int32_t* acc_out,
                        hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    const bool large = use_large(m, n);
    if (yt == kBF16) {
        EpiDequant<true> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
        return large ? launch<OpI8, CfgLarge>(xq, wq, m, n, k, e, stream)
                     : launch<OpI8, CfgSmall>(xq, wq, m, n, k, e, stream);
    }
    EpiDequant<false> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
    return large ? launch<OpI8, CfgLarge>(xq, wq, m, n, k, e, stream)
                 : launch<OpI8, CfgSmall>(xq, wq, m, n, k, e, stream);
}

int64_t gemm_sse_slots(int64_t m, int64_t n) {
    if (use_large(m, n)) return ((m + 255) / 256) * ((n + 255) / 256);
    return ((m + 127) / 128) * ((n + 127) / 128);
}

hipError_t gemm_sse(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                    const float* act_scale, const float* w_scale, const float* yref, double* slots,
                    hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    EpiSSE e{act_scale, w_scale, yref, slots, m, n, 0.0f, 0.0};
    return use_large(m, n) ? launch<OpI8, CfgLarge>(xq, wq, m, n, k, e, stream)
                           : launch<OpI8, CfgSmall>(xq, wq, m, n, k, e, stream);
}

hipError_t ref_gemm(const void* x, int xt, const void* w, int wt, int64_t m, int64_t n, int64_t k, float* yref,
                    hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (xt == kBF16 && wt == kBF16) {
        EpiStoreF32 e{yref, m, n};
        const int8_t* A = (const int8_t*)x;
        const int8_t* B = (const int8_t*)w;
        return use_large(m, n) ? launch<OpBF16, CfgLarge>(A, B, m, n, 2 * k, e, stream)
                               : launch<OpBF16, CfgSmall>(A, B, m, n, 2 * k, e, stream);
    }
    if (xt == kF32 && wt == kF32) {
        const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
        ref_gemm_f32_kernel<<<grid, dim3(256), 0, stream>>>((const float*)x, (const float*)w, m, n, k, yref);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;  // mixed input types are rejected by the C ABI
}

hipError_t reduce_slots(const double* slots, int64_t per_group, int groups, double count, double* out,
                        hipStream_t stream) {
    reduce_slots_kernel<<<dim3((unsigned)groups), dim3(256), 0, stream>>>(slots, per_group, count, out);
    return hipGetLastError();
}

}  // namespace sqk
