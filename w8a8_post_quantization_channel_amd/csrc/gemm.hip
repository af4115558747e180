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
#include <cmath>
#include <type_traits>

#include "sq_device.h"
#include "sq_kernels.h"

namespace {

using sqd::u32x4;
using sqd::dma16;
using sqd::kOutOfRange;
using sqd::lds_addr;
using sqd::tile_rsrc;
using sqd::wait_vmcnt;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Matrix-core operations on one 16-byte-per-lane operand pair. S is the
// output tile edge: S = 32 -> 32x32 tile, 16 accumulators per lane, 32 bytes
// of K per instruction; S = 16 -> 16x16 tile, 4 accumulators per lane, 64
// bytes of K per instruction. (bf16: the same byte geometry, half the elements.)
struct OpI8 {
    static constexpr int KB = 32;  // bytes of K per lane-pair per instruction (16 bytes per lane)
    using frag_t = v4i;
    template <int S>
    using acc_t = typename std::conditional<S == 32, v16i, v4i>::type;
    template <int S>
    __device__ static __forceinline__ acc_t<S> mfma(const v4i& a, const v4i& b, const acc_t<S>& c) {
        if constexpr (S == 32)
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    }
};

struct OpBF16 {
    static constexpr int KB = 32;
    using frag_t = v4i;
    template <int S>
    using acc_t = typename std::conditional<S == 32, v16f, v4f>::type;
    template <int S>
    __device__ static __forceinline__ acc_t<S> mfma(const v4i& a, const v4i& b, const acc_t<S>& c) {
        if constexpr (S == 32)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                           c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                           c, 0, 0, 0);
    }
};

// OCP FP8 E4M3 x E4M3 -> fp32 on gfx950's v_mfma_f32_32x32x64_f8f6f4 (the
// scaled form with both scales 0 is the unscaled instruction): 32 bytes of K
// per lane, 32 x 32 x 64 per instruction, the same rate per byte as int8.
typedef int v8i __attribute__((ext_vector_type(8)));
struct OpF8 {
    static constexpr int KB = 64;
    using frag_t = v8i;
    template <int S>
    using acc_t = v16f;
    template <int S>
    __device__ static __forceinline__ acc_t<S> mfma(const v8i& a, const v8i& b, const acc_t<S>& c) {
        static_assert(S == 32, "32 x 32 tiles only");
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

// 32-bit patterns of accumulator elements (taken by value: element access on
// a vector is not an addressable object)
__device__ __forceinline__ int as_bits(int v) { return v; }
__device__ __forceinline__ int as_bits(float v) { return __float_as_int(v); }
template <class E>
__device__ __forceinline__ E from_bits(int v) {
    if constexpr (std::is_same<E, float>::value)
        return __int_as_float(v);
    else
        return v;
}

// Row of accumulator element v within an S x S output tile, relative to the
// lane's first row (lane/32*4 for S = 32, lane/16*4 for S = 16); the column is
// lane % S.
template <int S>
__device__ __forceinline__ int acc_row(int v) {
    if constexpr (S == 32)
        return 8 * (v >> 2) + (v & 3);
    else
        return v;
}

constexpr int kBK = 128;  // bytes of K per LDS stage

// ---- epilogues ------------------------------------------------------------
// Each epilogue sees one S x S accumulator tile per call: the lane owns column
// `col` and the rows row0 + acc_row<S>(v) for its accumulator elements v.

// y = fp32(fp32(acc) * fp32(act_scale * w_scale[col])), fp32 or bf16 store;
// the raw int32 accumulator is stored too when acc_out is set. kH: both
// scales are stored as binary16 (ADR-010 "Consequences") and decoded
// (exactly) before the merge.
template <bool kBF16Out, class AccT = int32_t, bool kH = false>
struct EpiDequant {
    const void* act_scale;
    const void* w_scale;
    void* y;
    AccT* acc_out;
    int64_t M, N;
    float a;
    __device__ float ws(int64_t c) const {
        if constexpr (kH)
            return sqd::f16_dec(((const uint16_t*)w_scale)[c]);
        else
            return ((const float*)w_scale)[c];
    }
    __device__ void begin() {
        if constexpr (kH)
            a = sqd::f16_dec(*(const uint16_t*)act_scale);
        else
            a = *(const float*)act_scale;
    }
    template <int S, class Acc>
    __device__ void tile(const Acc& acc, int64_t row0, int64_t col) {
        if (col >= N) return;
        const float c = __fmul_rn(a, ws(col));
#pragma unroll
        for (int v = 0; v < S * S / 64; ++v) {
            const int64_t row = row0 + acc_row<S>(v);
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
    // one output element (the vector-ALU decode kernel)
    __device__ void one(AccT v, int64_t row, int64_t col) {
        if (row >= M || col >= N) return;
        const float val = __fmul_rn((float)v, __fmul_rn(a, ws(col)));
        const int64_t idx = row * N + col;
        if constexpr (kBF16Out)
            ((uint16_t*)y)[idx] = (uint16_t)sqd::f32_to_bf16_bits(val);
        else
            ((float*)y)[idx] = val;
        if (acc_out) acc_out[idx] = v;
    }
    // Eight consecutive columns col .. col + 7 (col % 8 == 0) owned by one
    // lane for a run of rows: their merged scales are loaded once.
    struct Cols {
        float c[8];
        int64_t col;
    };
    __device__ Cols cols8(int64_t col) {
        Cols cc;
        cc.col = col;
        if constexpr (kH) {
            if (col + 8 <= N) {  // eight binary16 scales: one 16-byte load (col % 8 == 0)
                const u32x4 h = *(const u32x4*)((const uint16_t*)w_scale + col);
                const uint32_t d[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    cc.c[2 * k] = __fmul_rn(a, sqd::f16_dec((uint16_t)(d[k] & 0xffffu)));
                    cc.c[2 * k + 1] = __fmul_rn(a, sqd::f16_dec((uint16_t)(d[k] >> 16)));
                }
                return cc;
            }
        } else if (col + 8 <= N && N % 4 == 0) {
            const float* w = (const float*)w_scale;
            const v4f s0 = *(const v4f*)(w + col), s1 = *(const v4f*)(w + col + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                cc.c[k] = __fmul_rn(a, s0[k]);
                cc.c[k + 4] = __fmul_rn(a, s1[k]);
            }
            return cc;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) cc.c[k] = col + k < N ? __fmul_rn(a, ws(col + k)) : 0.0f;
        return cc;
    }
    // fast: the caller's whole tile lies inside M x N and N % 8 == 0 (a
    // uniform condition), so no bounds checks and 16-byte stores
    __device__ void row8(const AccT (&acc)[8], int64_t row, const Cols& cc, bool fast) {
        const int64_t col = cc.col;
        float val[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) val[k] = __fmul_rn((float)acc[k], cc.c[k]);
        const int64_t idx = row * N + col;
        if (fast) {
            if constexpr (kBF16Out) {
                // y is zero or a nonzero integer times a * ws >= 6e-20
                // (a >= 1e-10 / 127, ws >= 1e-5 / 127; binary16 scales are
                // >= 2^-24 each): never subnormal, so the hardware rounding
                // equals f32_to_bf16_bits here
                u32x4 o;
                o.x = sqd::pack_bf16x2(val[0], val[1]);
                o.y = sqd::pack_bf16x2(val[2], val[3]);
                o.z = sqd::pack_bf16x2(val[4], val[5]);
                o.w = sqd::pack_bf16x2(val[6], val[7]);
                *(u32x4*)((uint16_t*)y + idx) = o;
            } else {
                *(v4f*)((float*)y + idx) = v4f{val[0], val[1], val[2], val[3]};
                *(v4f*)((float*)y + idx + 4) = v4f{val[4], val[5], val[6], val[7]};
            }
            if (acc_out) {
                *(v4i*)(acc_out + idx) = v4i{as_bits(acc[0]), as_bits(acc[1]), as_bits(acc[2]), as_bits(acc[3])};
                *(v4i*)(acc_out + idx + 4) = v4i{as_bits(acc[4]), as_bits(acc[5]), as_bits(acc[6]), as_bits(acc[7])};
            }
            return;
        }
        if (row >= M) return;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (col + k < N) {
                if constexpr (kBF16Out)
                    ((uint16_t*)y)[idx + k] = (uint16_t)sqd::f32_to_bf16_bits(val[k]);
                else
                    ((float*)y)[idx + k] = val[k];
                if (acc_out) acc_out[idx + k] = acc[k];
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
    template <int S, class Acc>
    __device__ void tile(const Acc& acc, int64_t row0, int64_t col) {
        if (col >= N) return;
        const float c = __fmul_rn(a, w_scale[col]);
#pragma unroll
        for (int v = 0; v < S * S / 64; ++v) {
            const int64_t row = row0 + acc_row<S>(v);
            if (row < M) {
                const float val = __fmul_rn((float)acc[v], c);
                const double d = (double)val - (double)yref[row * N + col];
                sum += d * d;
            }
        }
    }
    struct Cols {
        float c[8];
        int64_t col;
    };
    __device__ Cols cols8(int64_t col) {
        Cols cc;
        cc.col = col;
#pragma unroll
        for (int k = 0; k < 8; ++k) cc.c[k] = col + k < N ? __fmul_rn(a, w_scale[col + k]) : 0.0f;
        return cc;
    }
    // fast (the tile lies inside M x N, N % 8 == 0) and yref 16-byte aligned:
    // two 16-byte loads of the reference, and the eight squared errors added
    // as a fixed pairwise tree before they join the running sum (a short
    // dependency chain; the order is still the same on every run)
    __device__ void row8(const int (&acc)[8], int64_t row, const Cols& cc, bool fast) {
        if (fast && ((uintptr_t)yref & 15u) == 0) {
            const float* yr = yref + row * N + cc.col;
            const v4f r0 = *(const v4f*)yr, r1 = *(const v4f*)(yr + 4);
            const float ref[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
            double q[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const double d = (double)__fmul_rn((float)acc[k], cc.c[k]) - (double)ref[k];
                q[k] = d * d;
            }
            sum += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
            return;
        }
        if (row >= M) return;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (cc.col + k < N) {
                const float val = __fmul_rn((float)acc[k], cc.c[k]);
                const double d = (double)val - (double)yref[row * N + cc.col + k];
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
    template <int S, class Acc>
    __device__ void tile(const Acc& acc, int64_t row0, int64_t col) {
        if (col >= N) return;
#pragma unroll
        for (int v = 0; v < S * S / 64; ++v) {
            const int64_t row = row0 + acc_row<S>(v);
            if (row < M) y[row * N + col] = (float)acc[v];
        }
    }
    struct Cols {
        int64_t col;
    };
    __device__ Cols cols8(int64_t col) { return Cols{col}; }
    __device__ void row8(const float (&acc)[8], int64_t row, const Cols& cc, bool fast) {
        const int64_t col = cc.col;
        const int64_t idx = row * N + col;
        if (fast) {
            *(v4f*)(y + idx) = v4f{acc[0], acc[1], acc[2], acc[3]};
            *(v4f*)(y + idx + 4) = v4f{acc[4], acc[5], acc[6], acc[7]};
            return;
        }
        if (row >= M) return;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (col + k < N) y[idx + k] = acc[k];
    }
    __device__ void end(char*) {}
};

// ---- main kernel ------------------------------------------------------------

template <class Op, int BM, int BN, int WM, int WN, int S, class Epi>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_kernel(const int8_t* __restrict__ A,
                                                                         const int8_t* __restrict__ B,
                                                                         int64_t M, int64_t N, int64_t Kb,
                                                                         int tiles_m, int tiles_n, Epi epi) {
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    constexpr int ROWS = BM + BN;
    // 16-byte chunks per thread per stage (the last round may be partial)
    constexpr int CPT = (ROWS * (kBK / 16) + NT - 1) / NT;
    constexpr bool kExact = ROWS * (kBK / 16) % NT == 0;
    static_assert(S == 16 || S == 32, "matrix-core tile edge");
    static_assert(WM % S == 0 && WN % S == 0, "wave tile must hold whole MFMA tiles");
    constexpr int TM = WM / S, TN = WN / S;
    constexpr int KSTEP = S == 32 ? 32 : 64;  // bytes of K per MFMA
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
    bool live[CPT];  // chunk lies inside the stage
    int ldst[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int row = (tid >> 3) + c * (NT / 8);
        live[c] = kExact || row < ROWS;
        int64_t grow;
        const int8_t* base;
        if (!live[c]) {
            grow = 0;
            ok[c] = false;
            base = A;
        } else if (row < BM) {
            grow = m0 + row;
            ok[c] = grow < M;
            base = A;
        } else {
            grow = n0 + (row - BM);
            ok[c] = grow < N;
            base = B;
        }
        gsrc[c] = (const char*)base + (ok[c] ? grow * Kb : 0) + kcb;
        ldst[c] = live[c] ? row * kBK + ((kc ^ (row & 7)) << 4) : 0;
    }

    using Acc = typename Op::template acc_t<S>;
    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{};

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
        for (int c = 0; c < CPT; ++c)
            if (live[c]) *(u32x4*)(lds + buf * STAGE + ldst[c]) = stg[c];
    };
    // fragment reads: lane -> (row lane % S, 16-byte K chunk lane / S within
    // the instruction's K step); the physical chunk is XOR-swizzled by row & 7
    const int frag_row = lane & (S - 1);
    const int chunk_lane = lane / S;
    auto compute = [&](int buf) {
        const char* sa = lds + buf * STAGE + (wm * WM + frag_row) * kBK;
        const char* sb = lds + buf * STAGE + (BM + wn * WN + frag_row) * kBK;
#pragma unroll
        for (int ks = 0; ks < kBK / KSTEP; ++ks) {
            const int chunk = (((KSTEP / 16) * ks + chunk_lane) ^ (lane & 7)) << 4;
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const v4i*)(sa + i * S * kBK + chunk);
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = *(const v4i*)(sb + j * S * kBK + chunk);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Op::template mfma<S>(af[i], bf[j], acc[i][j]);
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
    const int64_t rbase = m0 + wm * WM + 4 * chunk_lane;
    const int64_t cbase = n0 + wn * WN + frag_row;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) epi.template tile<S>(acc[i][j], rbase + i * S, cbase + j * S);
    epi.end(lds);
}

// ---- direct-to-LDS pipelined kernel (large problems) ---------------------------
//
// Block tile 256 x BN (BN = 32 * TN), four waves, wave w owning output rows
// [64w, 64w + 64) x all BN columns: 2 x TN accumulators of 32 x 32 (int32, in
// AGPRs), one wave per SIMD. K advances in 128-byte steps through a ring of
// NS LDS stages (three when they fit in LDS, else two) filled by
// buffer_load ... lds (global -> LDS without VGPRs): the loads for step
// k + NS - 1 are issued while step k is multiplied.
//
// A step moves whole 128-byte row segments: every 128-byte cache line fetched
// from L2 is used in full by one instruction. (With 64-byte steps each request
// used half a line and the L2 -> LDS stream alone ran at about 60% of this
// rate.) Rows of A or B beyond M or N lie outside the per-tile buffer
// descriptor and read as zero; when k is an odd multiple of 64 bytes the upper
// half of the last step is redirected out of range too, so it reads as zero.
//
// LDS stage layout: rows of 128 bytes (A rows 0..255, then B rows), 16-byte
// chunk c of row r stored at position c ^ ((r >> 1) & 7). LDS has 64 banks of
// 4 bytes, so a 128-byte row covers half of them and rows r, r + 1 cover all;
// with this swizzle the 16 rows read by 16 lanes of one fragment read (lane l:
// row l % 32, chunk 2*substep + l / 32) land on 16 different 16-byte bank
// groups. One load instruction fills 8 consecutive rows (1 KB; lane q ->
// bytes 16q..16q+15, i.e. row q/8, position q%8), so lane q fetches logical
// chunk (q % 8) ^ ((row >> 1) & 7) of its row.
//
// Each step is a fixed instruction stream: MFMAs with the fragment reads of the
// next substep and the loads of a later step interleaved between them, and
// one barrier per step that publishes the next stage after an explicit vmcnt
// wait.

constexpr int kDmaBK = 128;     // bytes of K per stage
constexpr int kDmaBM = 256;     // rows of A per tile (4 waves x 64)
constexpr int kLdsBytes = 160 * 1024;

// LDS rings of the pipelined tile. Up to 256 x 160, three joint stages (the
// A rows, then the B rows, 128 bytes of K each) fit in the 160 KB. Wider
// tiles split the rings: one panel keeps three stages and the other two, so
// the loads of the first run two steps ahead and those of the second one.
template <int TN>
struct DmaRing {
    static constexpr int SA = kDmaBM * kDmaBK, SB = 32 * TN * kDmaBK;  // bytes per stage
    static constexpr bool kJoint = 3 * (SA + SB) <= kLdsBytes;
    static constexpr bool kDeepA = false;  // split rings: B (the weight panel) three stages deep
    static constexpr int NSA = kJoint || kDeepA ? 3 : 2, NSB = kJoint || !kDeepA ? 3 : 2;
    static constexpr int bytes = NSA * SA + NSB * SB;
    static_assert(bytes <= kLdsBytes, "the rings fit in LDS");
};

// XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD takes a
// contiguous range of tiles (b < ntiles maps onto every tile exactly once)
__device__ __forceinline__ int xcd_tile(int b, int ntiles) {
    const int xcd = b & 7, slot = b >> 3;
    const int per = ntiles >> 3, rem = ntiles & 7;
    return xcd * per + min(xcd, rem) + slot;
}

template <int TN>
constexpr int dma_lds_bytes() {
    return DmaRing<TN>::bytes;
}

// One 256 x 32*TN output tile; t is the tile's index after the XCD remap.
template <class Op, int TN, class Epi>
__device__ __forceinline__ void dma_tile(const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t M,
                                         int64_t N, int64_t Kb, int tiles_m, int tiles_n, int t, Epi& epi,
                                         char* lds) {
    using R = DmaRing<TN>;
    constexpr bool JOINT = R::kJoint;
    constexpr int BM = kDmaBM, BN = 32 * TN;
    constexpr int L = (BM + BN) / 32;                // 1 KB loads per wave per step
    constexpr int LA = BM / 32, LB = L - LA;         // ... of A rows, of B rows
    constexpr int NFA = 2, NFB = TN, NF = NFA + NFB; // fragment reads per substep
    constexpr int NMMA = 2 * TN;                     // MFMAs per substep
    constexpr int NSUB = kDmaBK / Op::KB;            // MFMA substeps per step
    constexpr bool DEEPA = R::kDeepA;
    // loads a step leaves in flight when it publishes the next one: those of
    // the step after next (every row with joint stages, the deep ring's rows
    // with split rings)
    constexpr int AHEAD = JOINT ? L : DEEPA ? LA : LB;
    static_assert(NF <= NMMA + 2, "fragment reads interleave with the MFMAs");
    static_assert(AHEAD < 64, "vmcnt range");
    static_assert(4 * 32 * BN * 4 <= R::bytes, "the epilogue transpose fits in the rings");
    // byte offsets of A stage s and B stage s
    constexpr auto aoff = [](int s) { return (uint32_t)(JOINT ? s * (R::SA + R::SB) : s * R::SA); };
    constexpr auto boff = [](int s) {
        return (uint32_t)(JOINT ? s * (R::SA + R::SB) + R::SA : R::NSA * R::SA + s * R::SB);
    };

    const int lane = threadIdx.x & 63;
    // the wave index is uniform across the wave; saying so keeps the load
    // descriptors and LDS destinations in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // tiles are grouped 4 tile-rows at a time so an XCD's range of tiles
    // covers a compact block of the output (shared A and B panels in L2)
    constexpr int GM = 4;
    const int group = t / (GM * tiles_n), in_group = t % (GM * tiles_n);
    const int group_rows = min(GM, tiles_m - group * GM);
    const int tm = group * GM + in_group % group_rows, tn = in_group / group_rows;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    // epilogue geometry: after the transpose, lane -> (row lane / G8 of each
    // round, eight-column group lane % G8); its scales are fetched now so
    // their latency hides under the main loop
    constexpr int G8 = BN / 8;     // eight-column groups per row
    constexpr int RPI = 64 / G8;   // rows per read-back round
    constexpr int ROUNDS = (32 + RPI - 1) / RPI;
    const int q = lane % G8, rsub = lane / G8;
    const bool active = lane < RPI * G8;
    epi.begin();
    const auto cc = epi.cols8(n0 + 8 * q);

    const v4i ra = tile_rsrc(A + m0 * Kb, min<int64_t>(BM, M - m0), Kb);
    const v4i rb = tile_rsrc(B + n0 * Kb, min<int64_t>(BN, N - n0), Kb);

    // load j of wave w fills rows [8 (4j + w), 8 (4j + w) + 8) of the A stage
    // (j < LA), or rows [8 (4(j - LA) + w), ...) of the B stage
    // row = 8 (4j + wave) + lane / 8, so (row >> 1) & 7 = (4 (wave & 1) + lane / 16) & 7 for every j
    const int chunk = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    int voff[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int row = (4 * j + wave) * 8 + (lane >> 3);
        voff[j] = (j < LA ? row : row - BM) * (int)Kb + chunk * 16;
    }
    const int64_t nk = (Kb + kDmaBK - 1) / kDmaBK;
    // k an odd multiple of 64 bytes: chunks 4..7 of the last step lie past k
    const bool half_tail = (Kb % kDmaBK) != 0;
    const bool hi_chunk = chunk >= 4;
    // stages are addressed by byte offset into lds (uniform values updated
    // each step, so fragment addresses are one VGPR per substep plus an
    // immediate offset)
    // load j of step kstep into A stage sa or B stage sb; `skip` (steps past
    // the end) reads zeros
    auto dma = [&](int j, uint32_t sa, uint32_t sb, int64_t kstep, bool skip) {
        const int soff = (int)(kstep * kDmaBK);
        const uint32_t dst = lds_addr(lds) + (j < LA ? sa + (uint32_t)(j * 4096) : sb + (uint32_t)((j - LA) * 4096)) +
                             (uint32_t)wave * 1024u;
        const bool cut = skip || (half_tail && kstep == nk - 1 && hi_chunk);
        dma16(j < LA ? ra : rb, dst, cut ? kOutOfRange : voff[j], soff);
    };

    using Acc = typename Op::template acc_t<32>;
    Acc acc[2][TN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{};

    // fragment addresses within a stage: row (lane % 32) of each 32-row block,
    // chunk 2*ks + lane/32 at position ^ (row & 7) = ^ (lane & 7)
    const int frow = lane & 31;
    const int c0 = (lane >> 5) ^ ((lane >> 1) & 7);  // chunk 2*ks + lane/32 lands at position c0 ^ 2*ks
    const int a_off = (wave * 64 + frow) * kDmaBK;
    const int b_off = frow * kDmaBK;
    using Frag = typename Op::frag_t;
    Frag fa[2][NFA], fb[2][NFB];  // [substep parity][tile]
    auto read_frag = [&](uint32_t sa, uint32_t sb, int ks, int f) {
        const char* pa = lds + sa;
        const char* pb = lds + sb;
        if constexpr (Op::KB == 32) {
            const int ch = (c0 ^ (2 * ks)) << 4;
            if (f < NFA)
                fa[ks & 1][f] = *(const v4i*)(pa + (a_off + ch) + f * 32 * kDmaBK);
            else
                fb[ks & 1][f - NFA] = *(const v4i*)(pb + (b_off + ch) + (f - NFA) * 32 * kDmaBK);
        } else {
            // 64 bytes of K per substep: lane (row, h) takes chunks 4ks + 2h and
            // 4ks + 2h + 1, stored at positions (chunk ^ ((row >> 1) & 7))
            const int sw = (lane >> 1) & 7, h2 = 2 * (lane >> 5);
            const int ch0 = ((4 * ks + h2) ^ sw) << 4, ch1 = ((4 * ks + h2 + 1) ^ sw) << 4;
            const char* p = f < NFA ? pa + a_off + f * 32 * kDmaBK : pb + b_off + (f - NFA) * 32 * kDmaBK;
            const v4i lo = *(const v4i*)(p + ch0), hi = *(const v4i*)(p + ch1);
            const Frag v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            if (f < NFA)
                fa[ks & 1][f] = v;
            else
                fb[ks & 1][f - NFA] = v;
        }
    };
    auto read_frags = [&](uint32_t sa, uint32_t sb, int ks) {
#pragma unroll
        for (int f = 0; f < NF; ++f) read_frag(sa, sb, ks, f);
    };
    auto publish = [&]() {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    };
    // stages of steps kb, kb + 1 and (three-deep rings) kb + 2
    uint32_t ca = aoff(0), na = aoff(1), fla = aoff(2);
    uint32_t cb = boff(0), nb = boff(1), flb = boff(2);
    // load o of step kb's issue order: joint stages, every row of step kb + 2
    // (A rows first); split rings, the shallow ring's rows of step kb + 1,
    // then the deep ring's rows of step kb + 2, so one in-order wait covers
    // both stages the next step reads
    auto load = [&](int o, int64_t kb) {
        if constexpr (JOINT) {
            dma(o, fla, fla + R::SA, kb + 2, !(kb + 2 < nk));
        } else if constexpr (DEEPA) {
            if (o < LB)
                dma(LA + o, 0, nb, kb + 1, !(kb + 1 < nk));
            else
                dma(o - LB, fla, 0, kb + 2, !(kb + 2 < nk));
        } else {
            if (o < LA)
                dma(o, na, 0, kb + 1, !(kb + 1 < nk));
            else
                dma(o, 0, flb, kb + 2, !(kb + 2 < nk));
        }
    };
    // prologue: step 0 and the rows of step 1 that run two steps ahead in
    // flight, then publish step 0
#pragma unroll
    for (int j = 0; j < L; ++j) dma(j, ca, cb, 0, false);
#pragma unroll
    for (int j = 0; j < L; ++j)
        if (JOINT || (DEEPA ? j < LA : j >= LA)) dma(j, na, JOINT ? na + R::SA : nb, 1, nk < 2);
    wait_vmcnt<AHEAD>();
    publish();
    read_frags(ca, cb, 0);

    // One step, in a fixed instruction order (sched_barrier between slots):
    // NSUB substeps of NMMA MFMAs; after MFMA m of a substep comes fragment
    // read m of the next substep (m < NF), and across the first NSUB - 1
    // substeps every DSTRIDE-th slot issues one of the step's L loads, so the
    // loads queue behind the matrix cores instead of stalling them. Before the
    // last substep: wait for step kb + 1 and publish it; the last substep
    // reads the first fragments of that stage (stale but in bounds after the
    // last step). Steps past the end load zeros, so every step has the same
    // instruction stream.
    constexpr int DSTRIDE = (NSUB - 1) * NMMA / L > 0 ? (NSUB - 1) * NMMA / L : 1;
    static_assert(Op::KB != 32 || (L - 1) * DSTRIDE < (NSUB - 1) * NMMA, "the loads fit in the first substeps");
    // 64-byte substeps (two per step): the L loads are dealt over the MFMA
    // slots of the first substep, one or two per slot
    constexpr int SLOTS1 = (NSUB - 1) * NMMA;
    for (int64_t kb = 0; kb < nk; ++kb) {
#pragma unroll
        for (int ks = 0; ks < NSUB; ++ks) {
            if (ks == NSUB - 1 && kb + 1 < nk) {
                wait_vmcnt<AHEAD>();
                publish();
            }
            const uint32_t rsa = ks + 1 < NSUB ? ca : na;
            const uint32_t rsb = JOINT ? rsa + R::SA : (ks + 1 < NSUB ? cb : nb);
            const int rks = (ks + 1) % NSUB;
#pragma unroll
            for (int m = 0; m < NMMA; ++m) {
                const int i = m / TN, j = m % TN;
                // W rows as the first operand: acc[i][j] is the transposed
                // 32 x 32 block (lane: one output row, four consecutive columns)
                acc[i][j] = Op::template mfma<32>(fb[ks & 1][j], fa[ks & 1][i], acc[i][j]);
                if (m < NF) read_frag(rsa, rsb, rks, m);
                const int slot = ks * NMMA + m;
                if constexpr (Op::KB == 32) {
                    if (ks + 1 < NSUB && slot % DSTRIDE == 0 && slot / DSTRIDE < L) load(slot / DSTRIDE, kb);
                } else {
#pragma unroll
                    for (int j = 0; j < L; ++j)
                        if (ks + 1 < NSUB && (j * SLOTS1) / L == slot) load(j, kb);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // rotate the rings (a two-deep ring swaps its stages)
        const uint32_t wa = ca, wb = cb;
        ca = na;
        na = R::NSA == 3 ? fla : wa;
        fla = wa;
        cb = nb;
        nb = R::NSB == 3 ? flb : wb;
        flb = wb;
    }
    wait_vmcnt<0>();  // zero-fill loads past the end may still be in flight

    // Epilogue: lane l holds, for row (l % 32) of each 32-row block i and
    // column block j, columns 8g + 4 (l / 32) + 0..3 in acc[i][j][4g .. 4g+3].
    // Each wave transposes one 32 x BN block at a time through its own LDS
    // area (16-byte chunk c of row r at position c ^ (r & 7)), then hands the
    // epilogue eight consecutive columns per lane for 16-byte row stores.
    __syncthreads();  // every wave is done with the stages
    using E = typename std::conditional<std::is_same<Op, OpI8>::value, int, float>::type;
    char* tw = lds + wave * (32 * BN * 4);
    const int h = lane >> 5;
    const bool fast = m0 + BM <= M && n0 + BN <= N && N % 8 == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = 8 * j + 2 * g + h;
                const Acc& t = acc[i][j];
                const v4i o = {as_bits(t[4 * g + 0]), as_bits(t[4 * g + 1]), as_bits(t[4 * g + 2]),
                               as_bits(t[4 * g + 3])};
                *(v4i*)(tw + frow * (BN * 4) + ((c ^ (frow & 7)) << 4)) = o;
            }
        auto rows = [&](int it, bool fast_rows) {
            const int r = it * RPI + rsub;
            if (!active || r >= 32) return;
            const v4i lo = *(const v4i*)(tw + r * (BN * 4) + (((2 * q) ^ (r & 7)) << 4));
            const v4i hi = *(const v4i*)(tw + r * (BN * 4) + (((2 * q + 1) ^ (r & 7)) << 4));
            const E v[8] = {from_bits<E>(lo.x), from_bits<E>(lo.y), from_bits<E>(lo.z), from_bits<E>(lo.w),
                            from_bits<E>(hi.x), from_bits<E>(hi.y), from_bits<E>(hi.z), from_bits<E>(hi.w)};
            epi.row8(v, m0 + wave * 64 + i * 32 + r, cc, fast_rows);
        };
        if (fast) {
#pragma unroll
            for (int it = 0; it < ROUNDS; ++it) rows(it, true);
        } else {
#pragma unroll 1
            for (int it = 0; it < ROUNDS; ++it) rows(it, false);
        }
    }
    __syncthreads();
    epi.end(lds);
}

template <class Op, int TN, class Epi>
__global__ __launch_bounds__(256) void gemm_dma_kernel(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                       int64_t M, int64_t N, int64_t Kb, int tiles_m, int tiles_n,
                                                       Epi epi) {
    __shared__ __attribute__((aligned(1024))) char lds[dma_lds_bytes<TN>()];
    dma_tile<Op, TN, Epi>(A, B, M, N, Kb, tiles_m, tiles_n, xcd_tile(blockIdx.x, tiles_m * tiles_n), epi, lds);
}

// Several products in one launch (the projections of a block): item i owns
// the blocks [first[i], first[i + 1]), a multiple of 8 apart, so a block's
// XCD and its tile are those of a launch of item i alone; blocks past the
// item's tile count return at once. The next product's tiles start as soon
// as compute units free up, instead of after the previous launch drains.
struct GemmTable {
    int count;
    int32_t first[sqk::kMaxBatch + 1];
    const int8_t* A[sqk::kMaxBatch];
    const int8_t* B[sqk::kMaxBatch];
    const void* act_scale[sqk::kMaxBatch];  // fp32, or binary16 (kH)
    const void* w_scale[sqk::kMaxBatch];    // fp32, or binary16 (kH)
    void* y[sqk::kMaxBatch];
    void* acc_out[sqk::kMaxBatch];  // int32 (int8 codes) or fp32 (e4m3 codes) accumulators, or NULL
    int64_t M[sqk::kMaxBatch], N[sqk::kMaxBatch], Kb[sqk::kMaxBatch];
    int32_t tiles_m[sqk::kMaxBatch], tiles_n[sqk::kMaxBatch];
    int32_t tn[sqk::kMaxBatch];  // the item's tile width / 32 (grouped launches with a second width)
};

template <class Op, int TN, bool kBF16Out, class AccT, bool kH, int TN2 = 0>
__global__ __launch_bounds__(256) void gemm_dma_grouped_kernel(const GemmTable tab) {
    __shared__ __attribute__((aligned(1024))) char
        lds[TN2 != 0 && dma_lds_bytes<TN2>() > dma_lds_bytes<TN>() ? dma_lds_bytes<TN2>() : dma_lds_bytes<TN>()];
    const int i = sqd::item_of(tab.first, tab.count, blockIdx.x);
    const int b = blockIdx.x - tab.first[i], ntiles = tab.tiles_m[i] * tab.tiles_n[i];
    if (b >= ntiles) return;
    using Epi = EpiDequant<kBF16Out, AccT, kH>;
    Epi epi{tab.act_scale[i], tab.w_scale[i], tab.y[i], (AccT*)tab.acc_out[i], tab.M[i], tab.N[i], 0.0f};
    if constexpr (TN2 != 0) {
        // items on the second (narrower) width: the launch's last products,
        // so that its final round of tiles drains more evenly
        if (tab.tn[i] == TN2) {
            dma_tile<Op, TN2, Epi>(tab.A[i], tab.B[i], tab.M[i], tab.N[i], tab.Kb[i], tab.tiles_m[i], tab.tiles_n[i],
                                   xcd_tile(b, ntiles), epi, lds);
            return;
        }
    }
    dma_tile<Op, TN, Epi>(tab.A[i], tab.B[i], tab.M[i], tab.N[i], tab.Kb[i], tab.tiles_m[i], tab.tiles_n[i],
                          xcd_tile(b, ntiles), epi, lds);
}

// The fp32 reference products of several bf16 activation batches (items of
// the table; act_scale, w_scale and acc_out unused): the plain fp32 store of
// the accumulator, every batch's tiles in one launch.
template <int TN>
__global__ __launch_bounds__(256) void ref_gemm_grouped_kernel(const GemmTable tab) {
    __shared__ __attribute__((aligned(1024))) char lds[dma_lds_bytes<TN>()];
    const int i = sqd::item_of(tab.first, tab.count, blockIdx.x);
    const int b = blockIdx.x - tab.first[i], ntiles = tab.tiles_m[i] * tab.tiles_n[i];
    if (b >= ntiles) return;
    EpiStoreF32 epi{(float*)tab.y[i], tab.M[i], tab.N[i]};
    dma_tile<OpBF16, TN, EpiStoreF32>(tab.A[i], tab.B[i], tab.M[i], tab.N[i], tab.Kb[i], tab.tiles_m[i],
                                      tab.tiles_n[i], xcd_tile(b, ntiles), epi, lds);
}

// ---- skinny kernel (decode: 4 < m <= 64) ------------------------------------------
//
// The product is bound by streaming the int8 weight once from HBM. A block of
// 4 waves owns BNR weight rows (16 or 48) and walks K in 512-byte chunks
// through NS LDS stages. A stage holds AR = max(16, MB) activation rows and
// the BNR weight rows, 512 bytes each, filled by buffer_load ... lds two rows
// per instruction (lanes 0-31 one row, 32-63 the next: four whole cache lines
// each). Loading the rows whole matters: measured on the 7B decode shapes, the
// same weight bytes read as 16 rows x 64 bytes per instruction (the MFMA
// fragment layout, straight into registers) stream at about two thirds of the
// rate. Activation rows >= MB are never loaded (they only feed output rows that
// are never stored); rows in [m, MB) and bytes past k read as zero. 16-byte
// chunk c of a row r sits at position c ^ (r & 15), so the 16 rows of a
// fragment read land in distinct banks. Wave w computes the 64-byte K steps w
// and w + 4 of each chunk with v_mfma_i32_16x16x64_i8 (lane l: row l % 16,
// bytes 16 (l / 16) .. +15 of the step, for both operands); the four waves'
// int32 partials are added through LDS at the end (exact in any order).
template <int MB, int BNR, int NS>
constexpr int skinny_lds_bytes() {
    return NS * ((MB < 16 ? 16 : MB) + BNR) * 512;
}

// the BNR weight rows from n0 of one product
template <int MB, int BNR, int NS, class Epi>
__device__ __forceinline__ void skinny_block(const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t M,
                                             int64_t N, int64_t Kb, Epi& epi, int64_t n0, char* lds) {
    constexpr int AR = MB < 16 ? 16 : MB, MT = AR / 16, NR = BNR / 16;
    constexpr int L = (MB + BNR) / 8;  // load instructions per wave per chunk (2 rows each)
    static_assert((MB + BNR) % 8 == 0 && MB % 2 == 0, "whole load rounds; a load's two rows on one side");
    constexpr int KC = 512, STAGE = (AR + BNR) * KC;
    static_assert(NS * STAGE <= 160 * 1024 && (NS - 2) * L < 64, "stages fit; vmcnt range");
    static_assert(4 * NR * MT * 64 * 16 <= NS * STAGE, "the partial sums fit in the stages");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nchunk = (Kb + KC - 1) / KC;
    const v4i ra = tile_rsrc(A, M, Kb);
    const v4i rb = tile_rsrc(B + n0 * Kb, min<int64_t>(BNR, N - n0), Kb);
    // load j of wave w fills loaded rows idx0 = 2 (4 j + w) and idx0 + 1:
    // activation rows while idx0 < MB, else weight rows idx0 - MB
    const int half = lane >> 5, pos = lane & 31;
    int voff[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int idx0 = 2 * (4 * j + wave);
        const int row = (idx0 < MB ? idx0 : idx0 - MB) + half;
        voff[j] = row * (int)Kb + ((pos ^ (row & 15)) << 4);
    }
    auto issue = [&](int64_t c, int stage) {
        const int soff = (int)(c * KC);
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int idx0 = __builtin_amdgcn_readfirstlane(2 * (4 * j + wave));
            const bool isa = idx0 < MB;
            const int row = (isa ? idx0 : idx0 - MB) + half;
            const bool cut = c * KC + ((pos ^ (row & 15)) << 4) >= Kb;  // past the end of the row
            const int srow0 = isa ? idx0 : AR + idx0 - MB;
            dma16(isa ? ra : rb, lds_addr(lds) + (uint32_t)(stage * STAGE + srow0 * KC), cut ? kOutOfRange : voff[j],
                  soff);
        }
    };
    v4i acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = v4i{0, 0, 0, 0};
    const int frow = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nchunk) issue(p, p);
    for (int64_t c = 0; c < nchunk; ++c) {
        // chunk c landed (NS - 2 younger chunks may be in flight, fewer at the end)
        if (c + NS - 2 < nchunk)
            wait_vmcnt<(NS - 2) * L>();
        else
            wait_vmcnt<0>();
        __syncthreads();  // ... for every wave; the stage read at chunk c - 1 is free
        if (c + NS - 1 < nchunk) issue(c + NS - 1, (int)((c + NS - 1) % NS));
        const char* st = lds + (c % NS) * STAGE;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int ch = ((4 * (wave + 4 * q) + kg) ^ frow) << 4;
            v4i a[MT], b[NR];
#pragma unroll
            for (int t = 0; t < MT; ++t) a[t] = *(const v4i*)(st + (16 * t + frow) * KC + ch);
#pragma unroll
            for (int r = 0; r < NR; ++r) b[r] = *(const v4i*)(st + (AR + 16 * r + frow) * KC + ch);
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b[r], acc[r][t], 0, 0, 0);
        }
    }
    __syncthreads();  // every wave is done with the stages
    v4i* part = (v4i*)lds;  // [wave][r][t][lane]
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) part[((wave * NR + r) * MT + t) * 64 + lane] = acc[r][t];
    __syncthreads();
    epi.begin();
    for (int rt = wave; rt < NR * MT; rt += 4) {
        const int r = rt / MT, t = rt % MT;
        v4i sum = part[(r * MT + t) * 64 + lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) sum += part[((w * NR + r) * MT + t) * 64 + lane];
        // 16x16 accumulator: lane holds column lane % 16, rows 4 (lane / 16) + v
        epi.template tile<16>(sum, 16 * t + 4 * (lane >> 4), n0 + 16 * r + (lane & 15));
    }
    __syncthreads();
    epi.end(lds);
}

template <int MB, int BNR, int NS, class Epi>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const int8_t* __restrict__ A,
                                                          const int8_t* __restrict__ B, int64_t M, int64_t N,
                                                          int64_t Kb, Epi epi) {
    __shared__ __attribute__((aligned(1024))) char lds[skinny_lds_bytes<MB, BNR, NS>()];
    skinny_block<MB, BNR, NS, Epi>(A, B, M, N, Kb, epi, (int64_t)blockIdx.x * BNR, lds);
}

// Several decode products in one launch: item i owns the blocks
// [first[i], first[i + 1]), one per BNR weight rows; the items share the
// activation-row class MB and the (BNR, NS) configuration.
template <int MB, int BNR, int NS, bool kBF16Out, bool kH>
__global__ __launch_bounds__(256) void gemm_skinny_grouped_kernel(const GemmTable tab) {
    __shared__ __attribute__((aligned(1024))) char lds[skinny_lds_bytes<MB, BNR, NS>()];
    const int i = sqd::item_of(tab.first, tab.count, blockIdx.x);
    using Epi = EpiDequant<kBF16Out, int32_t, kH>;
    Epi epi{tab.act_scale[i], tab.w_scale[i], tab.y[i], (int32_t*)tab.acc_out[i], tab.M[i], tab.N[i], 0.0f};
    skinny_block<MB, BNR, NS, Epi>(tab.A[i], tab.B[i], tab.M[i], tab.N[i], tab.Kb[i], epi,
                                   (int64_t)(blockIdx.x - tab.first[i]) * BNR, lds);
}

// ---- vector-ALU kernel (decode: m <= 4) -------------------------------------------
//
// At m <= 4 the product is the weight stream and nothing else, so it runs on
// the vector ALUs where every weight load can be fully coalesced: a block of 4
// waves owns kGemvR consecutive weight rows; wave w takes the 1 KB K chunks w,
// w + 4, w + 8, ... (CH chunks of them in flight per group); a lane holds 16
// bytes of each activation row per chunk and loads 16 contiguous bytes of each
// weight row per chunk (one wave instruction reads 1 KB of one row), and
// accumulates `v_dot4_i32_i8` products into one int32 per (weight row,
// activation row). The partials are added across the wave (DPP) and across
// the 4 waves (LDS): integer sums, exact in any order. (The 16-row MFMA tiles
// of the skinny kernel read 64 bytes of each of 16 rows per instruction and an
// activation fragment per weight fragment; measured on the 7B decode shapes at
// m = 1, this kernel takes 4.8 / 8.8 / 8.8 us where that one takes 5.5 / 11.2 /
// 12.8 us for 4096x4096 / 11008x4096 / 4096x11008, cold weights.)
constexpr int kGemvMaxM = 4;
constexpr int kGemvR = 4;    // weight rows per block
constexpr int kGemvCH = 4;   // most 1 KB chunks per wave in flight

// the kGemvR weight rows from r0 of one product
template <int MB, int CH, class Epi>
__device__ __forceinline__ void gemv_block(const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t M,
                                           int64_t N, int64_t Kb, Epi& epi, int64_t r0,
                                           int (&red)[4][kGemvR][MB]) {
    constexpr int R = kGemvR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nchunk = (Kb + 1023) / 1024;
    int acc[R][MB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = 0;
    for (int64_t c0 = wave; c0 < nchunk; c0 += 4 * CH) {
        v4i xv[CH][MB], wv[R][CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t kc = (c0 + 4 * c) * 1024 + 16 * lane;
            const bool in = c0 + 4 * c < nchunk && kc < Kb;
#pragma unroll
            for (int m = 0; m < MB; ++m) xv[c][m] = in && m < M ? *(const v4i*)(A + m * Kb + kc) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < R; ++r)
                wv[r][c] = in && r0 + r < N ? __builtin_nontemporal_load((const v4i*)(B + (r0 + r) * Kb + kc))
                                            : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < CH; ++c)
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    int t = acc[r][m];
                    t = __builtin_amdgcn_sdot4(wv[r][c].x, xv[c][m].x, t, false);
                    t = __builtin_amdgcn_sdot4(wv[r][c].y, xv[c][m].y, t, false);
                    t = __builtin_amdgcn_sdot4(wv[r][c].z, xv[c][m].z, t, false);
                    acc[r][m] = __builtin_amdgcn_sdot4(wv[r][c].w, xv[c][m].w, t, false);
                }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const int t = sqd::wave_sum(acc[r][m]);
            if (lane == 0) red[wave][r][m] = t;
        }
    __syncthreads();
    epi.begin();
    if (threadIdx.x < R * MB) {
        const int r = threadIdx.x / MB, m = threadIdx.x % MB;
        epi.one(red[0][r][m] + red[1][r][m] + red[2][r][m] + red[3][r][m], m, r0 + r);
    }
}

template <int MB, int CH, class Epi>
__global__ __launch_bounds__(256) void gemv_kernel(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                   int64_t M, int64_t N, int64_t Kb, Epi epi) {
    __shared__ int red[4][kGemvR][MB];
    gemv_block<MB, CH, Epi>(A, B, M, N, Kb, epi, (int64_t)blockIdx.x * kGemvR, red);
}

// Several products in one launch (the projections of a decode step that read
// their inputs at once: q, k and v, or gate and up): item i owns the blocks
// [first[i], first[i + 1]), one per kGemvR weight rows. The items share MB (at
// most MB activation rows each) and CH (the chunks in flight per wave); the
// launch ramps and drains once instead of once per product.
template <int MB, int CH, bool kBF16Out, bool kH>
__global__ __launch_bounds__(256) void gemv_grouped_kernel(const GemmTable tab) {
    __shared__ int red[4][kGemvR][MB];
    const int i = sqd::item_of(tab.first, tab.count, blockIdx.x);
    using Epi = EpiDequant<kBF16Out, int32_t, kH>;
    Epi epi{tab.act_scale[i], tab.w_scale[i], tab.y[i], (int32_t*)tab.acc_out[i], tab.M[i], tab.N[i], 0.0f};
    gemv_block<MB, CH, Epi>(tab.A[i], tab.B[i], tab.M[i], tab.N[i], tab.Kb[i], epi,
                            (int64_t)(blockIdx.x - tab.first[i]) * kGemvR, red);
}

template <class E>
struct IsDequant : std::false_type {};
template <bool kBF16Out, class AccT, bool kH>
struct IsDequant<EpiDequant<kBF16Out, AccT, kH>> : std::is_same<AccT, int32_t> {};

inline int gemv_rows(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

// chunks in flight per wave: those of the busiest wave, at most kGemvCH
inline int gemv_ch(int64_t Kb) {
    const int64_t per_wave = ((Kb + 1023) / 1024 + 3) / 4;
    return per_wave >= kGemvCH ? kGemvCH : (int)per_wave;
}

template <int MB, class Epi>
hipError_t launch_gemv_m(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                         hipStream_t stream) {
    const dim3 grid((unsigned)((N + kGemvR - 1) / kGemvR)), block(256);
    switch (gemv_ch(Kb)) {
        case 1: gemv_kernel<MB, 1, Epi><<<grid, block, 0, stream>>>(A, B, M, N, Kb, epi); break;
        case 2: gemv_kernel<MB, 2, Epi><<<grid, block, 0, stream>>>(A, B, M, N, Kb, epi); break;
        case 3: gemv_kernel<MB, 3, Epi><<<grid, block, 0, stream>>>(A, B, M, N, Kb, epi); break;
        default: gemv_kernel<MB, kGemvCH, Epi><<<grid, block, 0, stream>>>(A, B, M, N, Kb, epi); break;
    }
    return hipGetLastError();
}

template <class Epi>
hipError_t launch_gemv(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                       hipStream_t stream) {
    switch (gemv_rows(M)) {
        case 1: return launch_gemv_m<1>(A, B, M, N, Kb, epi, stream);
        case 2: return launch_gemv_m<2>(A, B, M, N, Kb, epi, stream);
        default: return launch_gemv_m<4>(A, B, M, N, Kb, epi, stream);
    }
}

// Tile configurations.
//   D256 / D224 / D192 / D160 / D128: the pipelined direct-to-LDS kernel,
//         256 x BN tiles (BN = 32 * TN); the width is chosen per problem so the
//         tile count fills the CUs in whole rounds (2048 x 5120 -> 256 tiles
//         of 256 x 160)
//   S128: the register-staged kernel, 128 x 128 tiles of 4 waves of 64 x 64
//         (small M or N)
template <int BM_, int BN_, int WM_, int WN_, int S_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_;
};
using CfgS128 = Cfg<128, 128, 64, 64, 32>;

enum TileCfg { kD256, kD224, kD192, kD160, kD128, kS128, kNumCfg, kK16 = kNumCfg };
constexpr int kCfgBM[kNumCfg + 1] = {256, 256, 256, 256, 256, 128, 64};
constexpr int kCfgBN[kNumCfg + 1] = {256, 224, 192, 160, 128, 128, 16};
// relative per-CU throughput of each tile shape, measured on MI355X on the
// Llama-2 70B MLP products (4096 tokens, many tiles per CU; TOPS normalised to
// 256 x 128): 256 x 256 with split rings leads by 11 %, the other widths are
// within 1 % of each other; used only to rank candidates
constexpr double kCfgEff[kNumCfg] = {1.11, 1.01, 1.00, 0.99, 1.00, 0.45};

template <class C>
constexpr int threads_of() {
    return (C::BM / C::WM) * (C::BN / C::WN) * 64;
}

int cu_count() {
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

// Pick the tiling with the least predicted time: (tile rounds over the CUs)
// x (tile area) / (per-CU efficiency of that tile shape). Up to 64 rows of
// activations (decode) the weight-streaming skinny kernel is used.
constexpr int64_t kSkinnyMaxM = 64;

TileCfg choose_cfg(int64_t M, int64_t N) {
    if (M <= kSkinnyMaxM) return kK16;
    const int64_t cus = cu_count();
    TileCfg best = kS128;
    double best_cost = 0.0;
    for (int c = 0; c < kNumCfg; ++c) {
        const int64_t tiles = ((M + kCfgBM[c] - 1) / kCfgBM[c]) * ((N + kCfgBN[c] - 1) / kCfgBN[c]);
        const int64_t rounds = (tiles + cus - 1) / cus;
        const double cost = (double)rounds * kCfgBM[c] * kCfgBN[c] / kCfgEff[c];
        if (c == 0 || cost < best_cost) {
            best_cost = cost;
            best = (TileCfg)c;
        }
    }
    return best;
}

int64_t tiles_of(TileCfg c, int64_t M, int64_t N) {
    return ((M + kCfgBM[c] - 1) / kCfgBM[c]) * ((N + kCfgBN[c] - 1) / kCfgBN[c]);
}

template <class Op, class C, class Epi>
hipError_t launch(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                  hipStream_t stream) {
    const int tiles_m = (int)((M + C::BM - 1) / C::BM);
    const int tiles_n = (int)((N + C::BN - 1) / C::BN);
    gemm_kernel<Op, C::BM, C::BN, C::WM, C::WN, C::S, Epi>
        <<<dim3((unsigned)(tiles_m * tiles_n)), dim3(threads_of<C>()), 0, stream>>>(A, B, M, N, Kb, tiles_m, tiles_n,
                                                                                   epi);
    return hipGetLastError();
}

template <class Op, int TN, class Epi>
hipError_t launch_dma(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                      hipStream_t stream) {
    const int tiles_m = (int)((M + kDmaBM - 1) / kDmaBM);
    const int tiles_n = (int)((N + 32 * TN - 1) / (32 * TN));
    gemm_dma_kernel<Op, TN, Epi>
        <<<dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, stream>>>(A, B, M, N, Kb, tiles_m, tiles_n, epi);
    return hipGetLastError();
}

// Skinny configurations (activation rows MB, weight rows per block BNR, LDS
// stages NS), measured on the 7B decode shapes with cold weights: many blocks
// (n >= 32 x compute units of 16 rows) favour two stages and more blocks per
// compute unit, few blocks four stages; at m > 32, wide outputs take 48 weight
// rows per block (the activation bytes per weight byte drop 3x). Epilogues
// other than the dequantization keep one block per 16 weight rows (the
// squared-error slots are counted that way).
template <int MB, class Epi>
hipError_t launch_skinny_mb(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                            hipStream_t stream) {
    const dim3 block(256);
    const unsigned b16 = (unsigned)((N + 15) / 16);
    if constexpr (MB == 64) {
        if (IsDequant<Epi>::value && N >= 8192) {
            gemm_skinny_kernel<64, 48, 2, Epi><<<dim3((unsigned)((N + 47) / 48)), block, 0, stream>>>(A, B, M, N, Kb, epi);
            return hipGetLastError();
        }
        gemm_skinny_kernel<64, 16, 3, Epi><<<dim3(b16), block, 0, stream>>>(A, B, M, N, Kb, epi);
        return hipGetLastError();
    } else {
        if (IsDequant<Epi>::value && b16 >= 2 * (unsigned)cu_count())
            gemm_skinny_kernel<MB, 16, 2, Epi><<<dim3(b16), block, 0, stream>>>(A, B, M, N, Kb, epi);
        else
            gemm_skinny_kernel<MB, 16, 4, Epi><<<dim3(b16), block, 0, stream>>>(A, B, M, N, Kb, epi);
        return hipGetLastError();
    }
}

template <class Epi>
hipError_t launch_skinny(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                         hipStream_t stream) {
    if (M <= 8) return launch_skinny_mb<8>(A, B, M, N, Kb, epi, stream);
    if (M <= 16) return launch_skinny_mb<16>(A, B, M, N, Kb, epi, stream);
    if (M <= 32) return launch_skinny_mb<32>(A, B, M, N, Kb, epi, stream);
    return launch_skinny_mb<64>(A, B, M, N, Kb, epi, stream);
}

template <class Op, class Epi>
hipError_t dispatch(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                    hipStream_t stream) {
    if constexpr (std::is_same<Op, OpI8>::value) {
        if constexpr (IsDequant<Epi>::value)
            if (M <= kGemvMaxM) return launch_gemv(A, B, M, N, Kb, epi, stream);
        if (M <= kSkinnyMaxM) return launch_skinny(A, B, M, N, Kb, epi, stream);
    }
    switch (choose_cfg(M, N)) {
        case kD256: return launch_dma<Op, 8>(A, B, M, N, Kb, epi, stream);
        case kD224: return launch_dma<Op, 7>(A, B, M, N, Kb, epi, stream);
        case kD192: return launch_dma<Op, 6>(A, B, M, N, Kb, epi, stream);
        case kD160: return launch_dma<Op, 5>(A, B, M, N, Kb, epi, stream);
        case kD128: return launch_dma<Op, 4>(A, B, M, N, Kb, epi, stream);
        default: return launch<Op, CfgS128>(A, B, M, N, Kb, epi, stream);  // S128, and bf16 at m <= 64
    }
}

// FP8 products: the pipelined kernel at every size (its tilings only), the
// width whose whole rounds of tiles cost least
int f8_cfg(int64_t M, int64_t N) {
    const int64_t cus = cu_count();
    int best = kD128;
    double best_cost = 0.0;
    for (int c = kD256; c <= kD128; ++c) {
        const int64_t rounds = (tiles_of((TileCfg)c, M, N) + cus - 1) / cus;
        const double cost = (double)rounds * kCfgBM[c] * kCfgBN[c] / kCfgEff[c];
        if (c == kD256 || cost < best_cost) {
            best_cost = cost;
            best = c;
        }
    }
    return best;
}

// Predicted duration of a grouped launch of the selected products at tiling
// c (in tile-area x 128-byte K steps / efficiency units): the tiles are dealt
// in launch order to the compute unit that frees first, as the dispatcher
// does, so one product's partial round fills with the next product's tiles.
// The units' free times are kept as at most kTimes (time, units) groups; past
// that a group joins the one nearest in time.
double group_time(const sqk::GemmItem* items, const bool* sel, int count, const int* cfg) {
    constexpr int kTimes = 16;
    double t[kTimes];
    int64_t u[kTimes];
    int ng = 1;
    t[0] = 0.0;
    u[0] = cu_count();
    for (int p = 0; p < count; ++p) {
        if (!sel[p]) continue;
        const int c = cfg[p];
        const double per = (double)kCfgBM[c] * kCfgBN[c] / kCfgEff[c];
        const double d = (double)((items[p].k + kDmaBK - 1) / kDmaBK) * per;
        int64_t left = tiles_of((TileCfg)c, items[p].m, items[p].n);
        while (left > 0) {
            int g = 0;
            for (int q = 1; q < ng; ++q)
                if (t[q] < t[g]) g = q;
            const int64_t take = std::min(left, u[g]);
            const double nt = t[g] + d;
            left -= take;
            u[g] -= take;
            if (u[g] == 0) {
                t[g] = t[ng - 1];
                u[g] = u[ng - 1];
                --ng;
            }
            int h = -1;
            for (int q = 0; q < ng; ++q)
                if (t[q] == nt) h = q;
            if (h < 0 && ng == kTimes) {
                h = 0;
                for (int q = 1; q < ng; ++q)
                    if (std::fabs(t[q] - nt) < std::fabs(t[h] - nt)) h = q;
            }
            if (h < 0) {
                t[ng] = nt;
                u[ng] = take;
                ++ng;
            } else {
                u[h] += take;
            }
        }
    }
    double end = 0.0;
    for (int q = 0; q < ng; ++q) end = std::max(end, t[q]);
    return end;
}

// The pipelined tiling of products that share one grouped launch: the width
// with the least predicted grouped time (for one product, the same choice as
// choose_cfg among the pipelined widths).
TileCfg group_cfg(const sqk::GemmItem* items, const bool* sel, int count) {
    TileCfg best = kD128;
    double best_t = 0.0;
    for (int c = kD256; c <= kD128; ++c) {
        int cfg[sqk::kMaxBatch];
        for (int p = 0; p < count; ++p) cfg[p] = c;
        const double t = group_time(items, sel, count, cfg);
        if (c == kD256 || t < best_t) {
            best_t = t;
            best = (TileCfg)c;
        }
    }
    return best;
}

// A launch on 256 x 256 tiles may run its last selected products on 256 x 128
// tiles (the kernel's second width), so that its final round of tiles drains
// more evenly: the number of last products to narrow (0 to 3) with the least
// predicted grouped time; cfg receives every selected item's tiling.
int group_tail(const sqk::GemmItem* items, const bool* sel, int count, TileCfg main, int* cfg) {
    for (int p = 0; p < count; ++p) cfg[p] = main;
    if (main != kD256) return 0;
    double best_t = group_time(items, sel, count, cfg);
    int best = 0;
    for (int j = 1; j <= 3; ++j) {
        int trial[sqk::kMaxBatch];
        int left = j, nsel = 0;
        for (int p = count - 1; p >= 0; --p) {
            trial[p] = main;
            if (sel[p]) {
                ++nsel;
                if (left > 0) {
                    trial[p] = kD128;
                    --left;
                }
            }
        }
        if (nsel <= j) break;  // at least one product keeps the main width
        const double t = group_time(items, sel, count, trial);
        if (t < best_t) {
            best_t = t;
            best = j;
        }
    }
    int left = best;
    for (int p = count - 1; p >= 0 && left > 0; --p)
        if (sel[p]) {
            cfg[p] = kD128;
            --left;
        }
    return best;
}

template <class Epi>
hipError_t dispatch_f8(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                       hipStream_t stream) {
    switch (f8_cfg(M, N)) {
        case kD256: return launch_dma<OpF8, 8>(A, B, M, N, Kb, epi, stream);
        case kD224: return launch_dma<OpF8, 7>(A, B, M, N, Kb, epi, stream);
        case kD192: return launch_dma<OpF8, 6>(A, B, M, N, Kb, epi, stream);
        case kD160: return launch_dma<OpF8, 5>(A, B, M, N, Kb, epi, stream);
        default: return launch_dma<OpF8, 4>(A, B, M, N, Kb, epi, stream);
    }
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

// TN2: a second tile width some items of the launch take (0: none)
template <class Op, class AccT, int TN, int TN2 = 0>
hipError_t launch_grouped(const GemmTable& tab, int64_t blocks, bool bf16, bool h, hipStream_t stream) {
    const dim3 grid((unsigned)blocks), block(256);
    if constexpr (std::is_same<Op, OpI8>::value) {
        if (h) {
            if (bf16)
                gemm_dma_grouped_kernel<Op, TN, true, AccT, true, TN2><<<grid, block, 0, stream>>>(tab);
            else
                gemm_dma_grouped_kernel<Op, TN, false, AccT, true, TN2><<<grid, block, 0, stream>>>(tab);
            return hipGetLastError();
        }
    } else if (h) {
        return hipErrorInvalidValue;  // binary16 scales are for int8 codes
    }
    if (bf16)
        gemm_dma_grouped_kernel<Op, TN, true, AccT, false, TN2><<<grid, block, 0, stream>>>(tab);
    else
        gemm_dma_grouped_kernel<Op, TN, false, AccT, false, TN2><<<grid, block, 0, stream>>>(tab);
    return hipGetLastError();
}

template <int MB, int CH>
void launch_gemv_grouped_ch(const GemmTable& tab, int64_t blocks, bool bf16, bool h, hipStream_t stream) {
    const dim3 grid((unsigned)blocks), block(256);
    if (h) {
        if (bf16) gemv_grouped_kernel<MB, CH, true, true><<<grid, block, 0, stream>>>(tab);
        else gemv_grouped_kernel<MB, CH, false, true><<<grid, block, 0, stream>>>(tab);
    } else {
        if (bf16) gemv_grouped_kernel<MB, CH, true, false><<<grid, block, 0, stream>>>(tab);
        else gemv_grouped_kernel<MB, CH, false, false><<<grid, block, 0, stream>>>(tab);
    }
}

template <int MB>
void launch_gemv_grouped_mb(const GemmTable& tab, int64_t blocks, int ch, bool bf16, bool h, hipStream_t stream) {
    switch (ch) {
        case 1: launch_gemv_grouped_ch<MB, 1>(tab, blocks, bf16, h, stream); break;
        case 2: launch_gemv_grouped_ch<MB, 2>(tab, blocks, bf16, h, stream); break;
        case 3: launch_gemv_grouped_ch<MB, 3>(tab, blocks, bf16, h, stream); break;
        default: launch_gemv_grouped_ch<MB, kGemvCH>(tab, blocks, bf16, h, stream); break;
    }
}

// the skinny kernel's configuration for an int8 product with the
// dequantizing epilogue (as launch_skinny_mb picks it)
struct SkinnyCfg {
    int mb, bnr, ns;
    bool operator==(const SkinnyCfg& o) const { return mb == o.mb && bnr == o.bnr && ns == o.ns; }
};
SkinnyCfg skinny_cfg(int64_t M, int64_t N) {
    const int mb = M <= 8 ? 8 : M <= 16 ? 16 : M <= 32 ? 32 : 64;
    if (mb == 64) return N >= 8192 ? SkinnyCfg{64, 48, 2} : SkinnyCfg{64, 16, 3};
    const int64_t b16 = (N + 15) / 16;
    return SkinnyCfg{mb, 16, b16 >= 2 * (int64_t)cu_count() ? 2 : 4};
}

template <int MB, int BNR, int NS>
void launch_skinny_grouped_cfg(const GemmTable& tab, int64_t blocks, bool bf16, bool h, hipStream_t stream) {
    const dim3 grid((unsigned)blocks), block(256);
    if (h) {
        if (bf16) gemm_skinny_grouped_kernel<MB, BNR, NS, true, true><<<grid, block, 0, stream>>>(tab);
        else gemm_skinny_grouped_kernel<MB, BNR, NS, false, true><<<grid, block, 0, stream>>>(tab);
    } else {
        if (bf16) gemm_skinny_grouped_kernel<MB, BNR, NS, true, false><<<grid, block, 0, stream>>>(tab);
        else gemm_skinny_grouped_kernel<MB, BNR, NS, false, false><<<grid, block, 0, stream>>>(tab);
    }
}

hipError_t launch_skinny_grouped(const GemmTable& tab, int64_t blocks, SkinnyCfg c, bool bf16, bool h,
                                 hipStream_t stream) {
    if (c == SkinnyCfg{64, 48, 2}) launch_skinny_grouped_cfg<64, 48, 2>(tab, blocks, bf16, h, stream);
    else if (c == SkinnyCfg{64, 16, 3}) launch_skinny_grouped_cfg<64, 16, 3>(tab, blocks, bf16, h, stream);
    else if (c == SkinnyCfg{32, 16, 2}) launch_skinny_grouped_cfg<32, 16, 2>(tab, blocks, bf16, h, stream);
    else if (c == SkinnyCfg{32, 16, 4}) launch_skinny_grouped_cfg<32, 16, 4>(tab, blocks, bf16, h, stream);
    else if (c == SkinnyCfg{16, 16, 2}) launch_skinny_grouped_cfg<16, 16, 2>(tab, blocks, bf16, h, stream);
    else if (c == SkinnyCfg{16, 16, 4}) launch_skinny_grouped_cfg<16, 16, 4>(tab, blocks, bf16, h, stream);
    else if (c == SkinnyCfg{8, 16, 2}) launch_skinny_grouped_cfg<8, 16, 2>(tab, blocks, bf16, h, stream);
    else if (c == SkinnyCfg{8, 16, 4}) launch_skinny_grouped_cfg<8, 16, 4>(tab, blocks, bf16, h, stream);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

int dma_width(TileCfg c) {
    switch (c) {
        case kD256: return 8;
        case kD224: return 7;
        case kD192: return 6;
        case kD160: return 5;
        case kD128: return 4;
        default: return 0;
    }
}

// The products that join item i's grouped launch: those not yet launched
// that take the pipelined tiles (their own choice is a pipelined width) and
// share its output type and scale storage; returns their common tiling, the
// one with the least predicted grouped time.
template <bool kF8>
TileCfg pipelined_group(const GemmItem* items, int count, int i, const bool* done, bool* sel) {
    auto width = [](const GemmItem& it) { return dma_width(kF8 ? (TileCfg)f8_cfg(it.m, it.n) : choose_cfg(it.m, it.n)); };
    const GemmItem& it = items[i];
    for (int j = 0; j < count; ++j) {
        const GemmItem& jt = items[j];
        sel[j] = j == i || (j > i && !done[j] && jt.m != 0 && jt.n != 0 && jt.yt == it.yt && jt.h == it.h &&
                            width(jt) != 0);
    }
    return group_cfg(items, sel, count);
}

// Products that take the pipelined tiles (and share the output type and
// scale storage) share one grouped launch, at one width for all of them; int8 products too small for the
// pipelined tiles run as single launches (FP8 products always take a
// pipelined width).
template <class Op, class AccT>
hipError_t gemm_batched_impl(const GemmItem* items, int count, hipStream_t stream) {
    constexpr bool kF8 = std::is_same<Op, OpF8>::value;
    auto width = [](const GemmItem& it) { return dma_width(kF8 ? (TileCfg)f8_cfg(it.m, it.n) : choose_cfg(it.m, it.n)); };
    bool done[kMaxBatch] = {};
    for (int i = 0; i < count; ++i) {
        if (done[i]) continue;
        done[i] = true;
        const GemmItem& it = items[i];
        if (it.m == 0 || it.n == 0) continue;
        const int tn = width(it);
        if constexpr (!kF8) {
            if (it.m <= kGemvMaxM) {
                // m <= 4: the vector-ALU kernel; products with the same row
                // class, chunks in flight, output type and scale storage share
                // one launch
                const int mb = gemv_rows(it.m), ch = gemv_ch(it.k);
                GemmTable tab{};
                int64_t blocks = 0;
                for (int j = i; j < count; ++j) {
                    const GemmItem& jt = items[j];
                    if (j > i && (done[j] || jt.m == 0 || jt.n == 0 || jt.m > kGemvMaxM || gemv_rows(jt.m) != mb ||
                                  gemv_ch(jt.k) != ch || jt.yt != it.yt || jt.h != it.h))
                        continue;
                    done[j] = true;
                    const int c = tab.count++;
                    tab.first[c] = (int32_t)blocks;
                    tab.A[c] = jt.xq;
                    tab.B[c] = jt.wq;
                    tab.act_scale[c] = jt.act_scale;
                    tab.w_scale[c] = jt.w_scale;
                    tab.y[c] = jt.y;
                    tab.acc_out[c] = jt.acc_out;
                    tab.M[c] = jt.m;
                    tab.N[c] = jt.n;
                    tab.Kb[c] = jt.k;
                    blocks += (jt.n + kGemvR - 1) / kGemvR;
                    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
                }
                tab.first[tab.count] = (int32_t)blocks;
                const bool bf16 = it.yt == kBF16;
                if (mb == 1) launch_gemv_grouped_mb<1>(tab, blocks, ch, bf16, it.h, stream);
                else if (mb == 2) launch_gemv_grouped_mb<2>(tab, blocks, ch, bf16, it.h, stream);
                else launch_gemv_grouped_mb<4>(tab, blocks, ch, bf16, it.h, stream);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                continue;
            }
        }
        if constexpr (!kF8) {
            // 4 < m <= 64: the skinny kernel. Products with the same
            // configuration, output type and scale storage share a launch,
            // except in the two-stage 16-row configuration (outputs of at
            // least 2 x CUs blocks on their own): measured on the 7B decode
            // shapes, q/k/v at m = 8-64 run 10-19 % faster in one launch, but
            // gate/up at m = 8-16, already that wide, 3-6 % slower.
            const SkinnyCfg cfg = skinny_cfg(it.m, it.n);
            if (it.m <= kSkinnyMaxM && !(cfg.bnr == 16 && cfg.ns == 2)) {
                GemmTable tab{};
                int64_t blocks = 0;
                for (int j = i; j < count; ++j) {
                    const GemmItem& jt = items[j];
                    if (j > i && (done[j] || jt.m == 0 || jt.n == 0 || jt.m <= kGemvMaxM || jt.m > kSkinnyMaxM ||
                                  !(skinny_cfg(jt.m, jt.n) == cfg) || jt.yt != it.yt || jt.h != it.h))
                        continue;
                    done[j] = true;
                    const int c = tab.count++;
                    tab.first[c] = (int32_t)blocks;
                    tab.A[c] = jt.xq;
                    tab.B[c] = jt.wq;
                    tab.act_scale[c] = jt.act_scale;
                    tab.w_scale[c] = jt.w_scale;
                    tab.y[c] = jt.y;
                    tab.acc_out[c] = jt.acc_out;
                    tab.M[c] = jt.m;
                    tab.N[c] = jt.n;
                    tab.Kb[c] = jt.k;
                    blocks += (jt.n + cfg.bnr - 1) / cfg.bnr;
                    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
                }
                tab.first[tab.count] = (int32_t)blocks;
                const hipError_t e = launch_skinny_grouped(tab, blocks, cfg, it.yt == kBF16, it.h, stream);
                if (e != hipSuccess) return e;
                continue;
            }
        }
        if (tn == 0) {  // the register-staged kernel: one launch per item
            hipError_t e = hipErrorInvalidValue;
            if constexpr (!kF8)
                e = gemm_dequant(it.xq, it.wq, it.m, it.n, it.k, it.act_scale, it.w_scale, it.y, it.yt,
                                 (int32_t*)it.acc_out, it.h, stream);
            if (e != hipSuccess) return e;
            continue;
        }
        bool sel[kMaxBatch] = {};
        int cfg[kMaxBatch];
        const TileCfg main = pipelined_group<kF8>(items, count, i, done, sel);
        const int gtn = dma_width(main);
        const bool mixed = group_tail(items, sel, count, main, cfg) > 0;
        GemmTable tab{};
        int64_t blocks = 0;
        for (int j = i; j < count; ++j) {
            if (!sel[j]) continue;
            const GemmItem& jt = items[j];
            done[j] = true;
            const int c = tab.count++;
            const int tnj = dma_width((TileCfg)cfg[j]);
            const int64_t tiles_m = (jt.m + kDmaBM - 1) / kDmaBM, tiles_n = (jt.n + 32 * tnj - 1) / (32 * tnj);
            tab.tn[c] = tnj;
            tab.first[c] = (int32_t)blocks;
            tab.A[c] = jt.xq;
            tab.B[c] = jt.wq;
            tab.act_scale[c] = jt.act_scale;
            tab.w_scale[c] = jt.w_scale;
            tab.y[c] = jt.y;
            tab.acc_out[c] = jt.acc_out;
            tab.M[c] = jt.m;
            tab.N[c] = jt.n;
            tab.Kb[c] = jt.k;
            tab.tiles_m[c] = (int32_t)tiles_m;
            tab.tiles_n[c] = (int32_t)tiles_n;
            blocks += (tiles_m * tiles_n + 7) / 8 * 8;  // whole XCD rounds per item
            if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        }
        tab.first[tab.count] = (int32_t)blocks;
        const bool bf16 = it.yt == kBF16;
        hipError_t e = hipErrorInvalidValue;
        switch (gtn) {
            case 8:
                e = mixed ? launch_grouped<Op, AccT, 8, 4>(tab, blocks, bf16, it.h, stream)
                          : launch_grouped<Op, AccT, 8>(tab, blocks, bf16, it.h, stream);
                break;
            case 7: e = launch_grouped<Op, AccT, 7>(tab, blocks, bf16, it.h, stream); break;
            case 6: e = launch_grouped<Op, AccT, 6>(tab, blocks, bf16, it.h, stream); break;
            case 5: e = launch_grouped<Op, AccT, 5>(tab, blocks, bf16, it.h, stream); break;
            case 4: e = launch_grouped<Op, AccT, 4>(tab, blocks, bf16, it.h, stream); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t gemm_dequant_batched(const GemmItem* items, int count, hipStream_t stream) {
    return gemm_batched_impl<OpI8, int32_t>(items, count, stream);
}

hipError_t gemm_fp8_batched(const GemmItem* items, int count, hipStream_t stream) {
    return gemm_batched_impl<OpF8, float>(items, count, stream);
}

hipError_t gemm_dequant(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                        const void* act_scale, const void* w_scale, void* y, int yt, int32_t* acc_out, bool h,
                        hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (h) {
        if (yt == kBF16) {
            EpiDequant<true, int32_t, true> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
            return dispatch<OpI8>(xq, wq, m, n, k, e, stream);
        }
        EpiDequant<false, int32_t, true> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
        return dispatch<OpI8>(xq, wq, m, n, k, e, stream);
    }
    if (yt == kBF16) {
        EpiDequant<true> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
        return dispatch<OpI8>(xq, wq, m, n, k, e, stream);
    }
    EpiDequant<false> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
    return dispatch<OpI8>(xq, wq, m, n, k, e, stream);
}

hipError_t gemm_fp8(const uint8_t* xq, const uint8_t* wq, int64_t m, int64_t n, int64_t k, const float* act_scale,
                    const float* w_scale, void* y, int yt, float* acc_out, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (yt == kBF16) {
        EpiDequant<true, float> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
        return dispatch_f8((const int8_t*)xq, (const int8_t*)wq, m, n, k, e, stream);
    }
    EpiDequant<false, float> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
    return dispatch_f8((const int8_t*)xq, (const int8_t*)wq, m, n, k, e, stream);
}

void gemm_tiling(int64_t m, int64_t n, int* block_m, int* block_n) {
    if (m <= kGemvMaxM) {  // the vector-ALU kernel: gemv_rows(m) activation rows x kGemvR weight rows
        *block_m = gemv_rows(m);
        *block_n = kGemvR;
        return;
    }
    if (m <= kSkinnyMaxM) {  // the skinny kernel: activation rows x weight rows per block
        *block_m = m <= 16 ? 16 : m <= 32 ? 32 : 64;
        *block_n = m > 32 && n >= 8192 ? 48 : 16;
        return;
    }
    const TileCfg c = choose_cfg(m, n);
    *block_m = kCfgBM[c];
    *block_n = kCfgBN[c];
}

void gemm_batched_tiling(const GemmItem* items, int count, int* block_m, int* block_n) {
    bool done[kMaxBatch] = {};
    for (int i = 0; i < count; ++i) {
        if (done[i]) continue;
        const GemmItem& it = items[i];
        if (it.m <= kSkinnyMaxM || it.n == 0 || choose_cfg(it.m, it.n) == kS128) {
            done[i] = true;
            gemm_tiling(it.m, it.n, &block_m[i], &block_n[i]);
            continue;
        }
        bool sel[kMaxBatch] = {};
        int cfg[kMaxBatch];
        group_tail(items, sel, count, pipelined_group<false>(items, count, i, done, sel), cfg);
        for (int j = i; j < count; ++j)
            if (sel[j]) {
                done[j] = true;
                block_m[j] = kCfgBM[cfg[j]];
                block_n[j] = kCfgBN[cfg[j]];
            }
    }
}

int64_t gemm_sse_slots(int64_t m, int64_t n) { return tiles_of(choose_cfg(m, n), m, n); }

hipError_t gemm_sse(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                    const float* act_scale, const float* w_scale, const float* yref, double* slots,
                    hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    EpiSSE e{act_scale, w_scale, yref, slots, m, n, 0.0f, 0.0};
    return dispatch<OpI8>(xq, wq, m, n, k, e, stream);
}

hipError_t ref_gemm(const void* x, int xt, const void* w, int wt, int64_t m, int64_t n, int64_t k, float* yref,
                    hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (xt == kBF16 && wt == kBF16) {
        EpiStoreF32 e{yref, m, n};
        return dispatch<OpBF16>((const int8_t*)x, (const int8_t*)w, m, n, 2 * k, e, stream);
    }
    if (xt == kF32 && wt == kF32) {
        const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
        ref_gemm_f32_kernel<<<grid, dim3(256), 0, stream>>>((const float*)x, (const float*)w, m, n, k, yref);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;  // mixed input types are rejected by the C ABI
}

hipError_t ref_gemm_batched(const void* const* x, int xt, int nb, int64_t rows, const void* w, int wt, int64_t n,
                            int64_t k, float* yref, hipStream_t stream) {
    if (nb <= 0 || rows == 0 || n == 0) return hipSuccess;
    // the grouped launch covers nb x (tiles of one batch): the tile width of
    // the whole problem
    const int tn = xt == kBF16 && wt == kBF16 ? dma_width(choose_cfg((int64_t)nb * rows, n)) : 0;
    if (tn == 0 || rows <= kSkinnyMaxM) {
        for (int b = 0; b < nb; ++b) {
            const hipError_t e = ref_gemm(x[b], xt, w, wt, rows, n, k, yref + (int64_t)b * rows * n, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int64_t tiles_m = (rows + kDmaBM - 1) / kDmaBM, tiles_n = (n + 32 * tn - 1) / (32 * tn);
    const int64_t per = (tiles_m * tiles_n + 7) / 8 * 8;  // whole XCD rounds per batch
    for (int b0 = 0; b0 < nb; b0 += kMaxBatch) {
        GemmTable tab{};
        int64_t blocks = 0;
        for (int b = b0; b < nb && b < b0 + kMaxBatch; ++b) {
            const int c = tab.count++;
            tab.first[c] = (int32_t)blocks;
            tab.A[c] = (const int8_t*)x[b];
            tab.B[c] = (const int8_t*)w;
            tab.y[c] = yref + (int64_t)b * rows * n;
            tab.M[c] = rows;
            tab.N[c] = n;
            tab.Kb[c] = 2 * k;
            tab.tiles_m[c] = (int32_t)tiles_m;
            tab.tiles_n[c] = (int32_t)tiles_n;
            blocks += per;
            if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        }
        tab.first[tab.count] = (int32_t)blocks;
        const dim3 grid((unsigned)blocks), block(256);
        switch (tn) {
            case 8: ref_gemm_grouped_kernel<8><<<grid, block, 0, stream>>>(tab); break;
            case 7: ref_gemm_grouped_kernel<7><<<grid, block, 0, stream>>>(tab); break;
            case 6: ref_gemm_grouped_kernel<6><<<grid, block, 0, stream>>>(tab); break;
            case 5: ref_gemm_grouped_kernel<5><<<grid, block, 0, stream>>>(tab); break;
            default: ref_gemm_grouped_kernel<4><<<grid, block, 0, stream>>>(tab); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t reduce_slots(const double* slots, int64_t per_group, int groups, double count, double* out,
                        hipStream_t stream) {
    reduce_slots_kernel<<<dim3((unsigned)groups), dim3(256), 0, stream>>>(slots, per_group, count, out);
    return hipGetLastError();
}

}  // namespace sqk
