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
#include <type_traits>

#include "sq_device.h"
#include "sq_kernels.h"

namespace {

using sqd::u32x4;

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
    template <int S, class Acc>
    __device__ void tile(const Acc& acc, int64_t row0, int64_t col) {
        if (col >= N) return;
        const float c = __fmul_rn(a, w_scale[col]);
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
// AGPRs), one wave per SIMD. K advances in 64-byte steps through a ring of
// four LDS stages filled by buffer_load ... lds (global -> LDS without
// VGPRs): the loads for step k + 3 are issued while step k is multiplied, so
// three steps of memory latency are hidden. Rows of A or B beyond M or N lie
// outside the per-tile buffer descriptor and read as zero; the stage is
// padded to a multiple of 64 rows (the padding rows are such out-of-range B
// rows) so every wave issues the same number of loads.
//
// LDS stage layout: rows of 64 bytes (A rows 0..255, then B rows), 16-byte
// chunk c of row r stored at position c ^ ((r >> 2) & 3): sixteen consecutive
// rows then cover all sixteen 16-byte bank groups, for any chunk. One load
// instruction fills 16 consecutive rows (1 KB, lane q -> bytes 16q..16q+15,
// i.e. row q/4, position q%4), so lane q fetches logical chunk
// (q % 4) ^ ((q >> 4) & 3) of its row. An MFMA fragment read (lane l: row
// l % 32, chunk 2*substep + l / 32) is then conflict-free.
//
// Each K step is one basic block in the steady state: the fragment reads for
// the next substep are interleaved one per MFMA (sched_group_barrier), and one
// barrier per step publishes the next stage after an explicit vmcnt wait.

constexpr int kDmaBK = 64;      // bytes of K per stage
constexpr int kDmaBM = 256;     // rows of A per tile (4 waves x 64)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Raw buffer descriptor (stride 0) over one tile's panel: offsets at or past
// num_records = valid bytes read as zero.
__device__ __forceinline__ v4i tile_rsrc(const int8_t* base, int64_t rows_valid, int64_t kb) {
    const uint64_t b = (uint64_t)base;
    v4i r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r.z = __builtin_amdgcn_readfirstlane((int)(rows_valid * kb));
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16*lane.
// Written as asm so that the only waits on these loads are the explicit
// s_waitcnt vmcnt(...) placed before the barriers that publish each stage
// (the compiler would otherwise drain every load in flight before reading
// any stage). No register receives the data.
__device__ __forceinline__ void dma16(const v4i& rsrc, uint32_t lds, int voff, int soff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// scheduling-group masks (LLVM AMDGPU)
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <class Op, int TN, class Epi>
__global__ __launch_bounds__(256) void gemm_dma_kernel(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                       int64_t M, int64_t N, int64_t Kb, int tiles_m, int tiles_n,
                                                       Epi epi) {
    constexpr int BM = kDmaBM, BN = 32 * TN;
    constexpr int ROWS = (BM + BN + 63) / 64 * 64;   // padded to whole load rounds
    constexpr int STAGE = ROWS * kDmaBK;
    constexpr int L = ROWS / 64;                     // 1 KB loads per wave per stage
    constexpr int NFA = 2, NFB = TN, NF = NFA + NFB; // fragment reads per substep
    constexpr int NMMA = 2 * TN;                     // MFMAs per substep
    static_assert(NF <= NMMA + 2, "fragment reads interleave with the MFMAs");
    __shared__ __attribute__((aligned(1024))) char st0[STAGE];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE];
    __shared__ __attribute__((aligned(1024))) char st2[STAGE];
    __shared__ __attribute__((aligned(1024))) char st3[STAGE];

    const int lane = threadIdx.x & 63;
    // the wave index is uniform across the wave; saying so keeps the load
    // descriptors and LDS destinations in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // tile order: each XCD (workgroup b runs on XCD b % 8) takes a contiguous
    // range of tiles, and tiles are grouped 4 tile-rows at a time so an XCD's
    // range covers a compact block of the output (shared A and B panels in L2)
    const int ntiles = tiles_m * tiles_n;
    int t = blockIdx.x;
    {
        const int xcd = t & 7, slot = t >> 3;
        const int per = ntiles >> 3, rem = ntiles & 7;
        t = xcd * per + min(xcd, rem) + slot;
    }
    constexpr int GM = 4;
    const int group = t / (GM * tiles_n), in_group = t % (GM * tiles_n);
    const int group_rows = min(GM, tiles_m - group * GM);
    const int tm = group * GM + in_group % group_rows, tn = in_group / group_rows;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const v4i ra = tile_rsrc(A + m0 * Kb, min<int64_t>(BM, M - m0), Kb);
    const v4i rb = tile_rsrc(B + n0 * Kb, min<int64_t>(BN, N - n0), Kb);

    // per-lane byte offset (within its panel) of each load this wave issues;
    // load j of wave w fills stage rows [16 (4j + w), 16 (4j + w) + 16), which
    // are A rows exactly when j < BM / 64
    static_assert(BM % 64 == 0, "A rows fill whole load rounds");
    int voff[L];
    uint32_t ldsoff[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int g = 4 * j + wave;
        const int row = g * 16 + (lane >> 2);
        const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
        voff[j] = (j * 64 < BM ? row : row - BM) * (int)Kb + chunk * 16;
        ldsoff[j] = (uint32_t)(g * 1024);
    }
    auto issue = [&](const char* stage, int64_t kstep) {
        const int soff = (int)(kstep * kDmaBK);
        const uint32_t base = lds_addr(stage);
#pragma unroll
        for (int j = 0; j < L; ++j) dma16(j * 64 < BM ? ra : rb, base + ldsoff[j], voff[j], soff);
    };

    using Acc = typename Op::template acc_t<32>;
    Acc acc[2][TN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{};

    // fragment addresses within a stage: row (lane % 32) of each 32-row block,
    // chunk 2*ks + lane/32 at position ^ ((row >> 2) & 3) = ^ ((lane >> 2) & 3)
    const int frow = lane & 31;
    const int sw = (lane >> 2) & 3;
    const int a_off = (wave * 64 + frow) * kDmaBK;
    const int b_off = (BM + frow) * kDmaBK;
    v4i fa[2][NFA], fb[2][NFB];  // [substep][tile]
    auto read_frag = [&](const char* stage, int ks, int f) {
        const int ch = ((2 * ks + (lane >> 5)) ^ sw) << 4;
        if (f < NFA)
            fa[ks][f] = *(const v4i*)(stage + a_off + f * 32 * kDmaBK + ch);
        else
            fb[ks][f - NFA] = *(const v4i*)(stage + b_off + (f - NFA) * 32 * kDmaBK + ch);
    };
    auto read_frags = [&](const char* stage, int ks) {
#pragma unroll
        for (int f = 0; f < NF; ++f) read_frag(stage, ks, f);
    };
    auto mma = [&](int ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = Op::template mfma<32>(fa[ks][i], fb[ks][j], acc[i][j]);
    };
    // MFMAs of substep `ks` with the NF reads of (stage, rks) interleaved
    auto mma_with_reads = [&](int ks, const char* stage, int rks) {
        read_frags(stage, rks);
        mma(ks);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMMA - NF > 0 ? NMMA - NF : 0, 0);
    };
    auto publish = [&]() {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    };

    const int64_t nk = Kb / kDmaBK;  // k is a multiple of 64 elements
    // prologue: steps 0..2 in flight, then publish step 0
    issue(st0, 0);
    if (nk > 1) issue(st1, 1);
    if (nk > 2) issue(st2, 2);
    if (nk > 2) wait_vmcnt<2 * L>();
    else if (nk > 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
    publish();
    read_frags(st0, 0);

    // steady state: step kb on stage S, with steps kb+1 .. kb+3 in range
    auto steady = [&](auto S_, int64_t kb) {
        constexpr int S = decltype(S_)::value;
        const char* cur = S == 0 ? st0 : S == 1 ? st1 : S == 2 ? st2 : st3;
        const char* nxt = S == 0 ? st1 : S == 1 ? st2 : S == 2 ? st3 : st0;
        const char* fill = S == 0 ? st3 : S == 1 ? st0 : S == 2 ? st1 : st2;
        issue(fill, kb + 3);
        mma_with_reads(0, cur, 1);
        wait_vmcnt<2 * L>();  // step kb+1 landed (for this wave); kb+2, kb+3 may fly
        publish();            // ... and for every wave
        mma_with_reads(1, nxt, 0);
    };
    // tail step: fewer than three steps ahead
    auto tail = [&](auto S_, int64_t kb) {
        constexpr int S = decltype(S_)::value;
        const char* cur = S == 0 ? st0 : S == 1 ? st1 : S == 2 ? st2 : st3;
        const char* nxt = S == 0 ? st1 : S == 1 ? st2 : S == 2 ? st3 : st0;
        read_frags(cur, 1);
        mma(0);
        if (kb + 1 < nk) {
            if (kb + 2 < nk) wait_vmcnt<L>();
            else wait_vmcnt<0>();
            publish();
            read_frags(nxt, 0);
        }
        mma(1);
    };
    int64_t kb = 0;
    for (; kb + 6 < nk; kb += 4) {
        steady(std::integral_constant<int, 0>{}, kb);
        steady(std::integral_constant<int, 1>{}, kb + 1);
        steady(std::integral_constant<int, 2>{}, kb + 2);
        steady(std::integral_constant<int, 3>{}, kb + 3);
    }
    // the remaining steps (at most six), stage = kb % 4 with kb % 4 == 0 here
    if (kb + 3 < nk) steady(std::integral_constant<int, 0>{}, kb++);
    else if (kb < nk) tail(std::integral_constant<int, 0>{}, kb++);
    if (kb + 3 < nk) steady(std::integral_constant<int, 1>{}, kb++);
    else if (kb < nk) tail(std::integral_constant<int, 1>{}, kb++);
    if (kb + 3 < nk) steady(std::integral_constant<int, 2>{}, kb++);
    else if (kb < nk) tail(std::integral_constant<int, 2>{}, kb++);
    if (kb < nk) tail(std::integral_constant<int, 3>{}, kb++);
    if (kb < nk) tail(std::integral_constant<int, 0>{}, kb++);
    if (kb < nk) tail(std::integral_constant<int, 1>{}, kb++);

    epi.begin();
    const int64_t rbase = m0 + wave * 64 + 4 * (lane >> 5);
    const int64_t cbase = n0 + frow;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) epi.template tile<32>(acc[i][j], rbase + i * 32, cbase + j * 32);
    __syncthreads();
    epi.end(st0);
}

// ---- skinny kernel (decode: m <= 64) -------------------------------------------
//
// The product is bound by streaming the int8 weight once from HBM. A block of
// eight waves owns 16 output columns (16 weight rows) and all of K; wave w
// takes every eighth 64-byte K step, so the eight waves read disjoint parts
// of the same rows and their int32 partials are summed in LDS in a fixed
// order (exact). v_mfma_i32_16x16x64_i8 with the m rows padded to 16 (MT
// tiles of 16 rows): lane l holds row l % 16 and bytes 16 (l / 16) .. +15 of
// a 64-byte K step, for both operands. Weight rows past n and activation rows
// past m are clamped to the last valid row: their outputs are never stored.
// Each lane keeps U K steps of weight bytes in flight.

constexpr int kSkinnyWaves = 8;

template <int MT, int U, class Epi>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny_kernel(const int8_t* __restrict__ A,
                                                                      const int8_t* __restrict__ B, int64_t M,
                                                                      int64_t N, int64_t Kb, Epi epi) {
    __shared__ v4i part[kSkinnyWaves][MT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t brow = min<int64_t>(n0 + (lane & 15), N - 1);
    const int kl = (lane >> 4) * 16;  // byte offset within a 64-byte K step
    const int8_t* bp = B + brow * Kb + kl;
    const int8_t* ap[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ap[t] = A + min<int64_t>(16 * t + (lane & 15), M - 1) * Kb + kl;

    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};

    const int64_t nsteps = Kb / 64;
    // K steps of this wave: wave, wave + 8, wave + 16, ...
    int64_t st = wave;
    for (; st + (int64_t)kSkinnyWaves * (U - 1) < nsteps; st += (int64_t)kSkinnyWaves * U) {
        v4i b[U], a[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t off = (st + (int64_t)u * kSkinnyWaves) * 64;
            b[u] = __builtin_nontemporal_load((const v4i*)(bp + off));
#pragma unroll
            for (int t = 0; t < MT; ++t) a[u][t] = *(const v4i*)(ap[t] + off);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][t], b[u], acc[t], 0, 0, 0);
    }
    for (; st < nsteps; st += kSkinnyWaves) {
        const int64_t off = st * 64;
        const v4i b = __builtin_nontemporal_load((const v4i*)(bp + off));
#pragma unroll
        for (int t = 0; t < MT; ++t)
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(*(const v4i*)(ap[t] + off), b, acc[t], 0, 0, 0);
    }

#pragma unroll
    for (int t = 0; t < MT; ++t) part[wave][t][lane] = acc[t];
    __syncthreads();
    epi.begin();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            v4i sum = part[0][t][lane];
#pragma unroll
            for (int w = 1; w < kSkinnyWaves; ++w) sum += part[w][t][lane];
            // 16x16 accumulator: lane holds column lane % 16, rows 4 (lane / 16) + v
            epi.template tile<16>(sum, 16 * t + 4 * (lane >> 4), n0 + (lane & 15));
        }
    }
    __syncthreads();
    epi.end((char*)part);
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
// relative per-CU throughput of each tile shape, measured on MI355X over the
// Llama-2 13B/70B prefill shapes (TOPS per busy CU, normalised to 256 x 192);
// used only to rank candidates
constexpr double kCfgEff[kNumCfg] = {0.82, 0.78, 1.00, 0.99, 0.88, 0.60};

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

template <int MT, class Epi>
hipError_t launch_skinny(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                         hipStream_t stream) {
    constexpr int U = MT == 1 ? 8 : 4;
    gemm_skinny_kernel<MT, U, Epi>
        <<<dim3((unsigned)((N + 15) / 16)), dim3(64 * kSkinnyWaves), 0, stream>>>(A, B, M, N, Kb, epi);
    return hipGetLastError();
}

template <class Op, class Epi>
hipError_t dispatch(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t Kb, Epi epi,
                    hipStream_t stream) {
    if constexpr (std::is_same<Op, OpI8>::value) {
        if (M <= kSkinnyMaxM) {
            if (M <= 16) return launch_skinny<1>(A, B, M, N, Kb, epi, stream);
            if (M <= 32) return launch_skinny<2>(A, B, M, N, Kb, epi, stream);
            return launch_skinny<4>(A, B, M, N, Kb, epi, stream);
        }
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
    if (yt == kBF16) {
        EpiDequant<true> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
        return dispatch<OpI8>(xq, wq, m, n, k, e, stream);
    }
    EpiDequant<false> e{act_scale, w_scale, y, acc_out, m, n, 0.0f};
    return dispatch<OpI8>(xq, wq, m, n, k, e, stream);
}

void gemm_tiling(int64_t m, int64_t n, int* block_m, int* block_n) {
    const TileCfg c = choose_cfg(m, n);
    *block_m = kCfgBM[c];
    *block_n = kCfgBN[c];
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

hipError_t reduce_slots(const double* slots, int64_t per_group, int groups, double count, double* out,
                        hipStream_t stream) {
    reduce_slots_kernel<<<dim3((unsigned)groups), dim3(256), 0, stream>>>(slots, per_group, count, out);
    return hipGetLastError();
}

}  // namespace sqk
