// quant.hip -- the two quantization passes of the SmoothQuant W8A8 layer.
//
// quant_weight: offline fold W' = W diag(s) (kwkr.cn blog §3.2) and symmetric
//   int8 with one scale per output row (ADR-010 "Context" item 3). Rows stream
//   through an LDS ring (global -> LDS loads running ahead of the math); the
//   threads of a block own fixed columns (their s values in registers) and
//   keep W' in registers between the row max and the quantize pass, so W is
//   read from HBM exactly once.
// quant_act: runtime x * (1/s) strictly before the per-tensor quantizer
//   (kwkr.cn blog §3.2 and §5.2; ADR-010 "Key design" items 4-5). A lane owns
//   one 16-byte column vector and keeps its inv_s values in registers while
//   the four waves of a block walk interleaved rows.
//
// The weight pass works on "groups" of 16 consecutive elements of a row (32
// bytes of bf16, 64 of fp32), which become 16 int8 codes: one 16-byte store.
#include <algorithm>
#include <type_traits>

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

// Weight rows streamed through LDS. A persistent block of WV waves walks
// "stages" of RB consecutive rows (a contiguous run of W), kept in a ring of NS
// LDS buffers filled by buffer_load ... lds, so the loads of the next stages
// fly while this one is reduced and quantized. The RB * kvec 16-byte vectors
// of a stage are dealt out flat: thread t takes vectors j = t, t + T, ...
// (T threads, at most NV each), so every thread has the same work whatever the
// row length; the row r_j = j / kvec and column c_j = j % kvec of each of its
// slots are fixed for a weight, and the thread keeps the s values of its
// columns in registers. Per stage: pass 1 forms W' = W * s in registers and
// the row maxima (a select per row, wave shuffles, one LDS exchange and
// barrier), pass 2 quantizes the registers and stores 4 or 8 codes per vector
// (the codes of a stage are as contiguous as its input). W is read from HBM
// once.
//
// One launch can cover several weights (the projections of a block): their
// stages are numbered one after the other, item i owning stages
// [first[i], first[i + 1]), and a block that moves on to the next item
// recomputes its slots and reloads its s registers.

struct QwTable {
    int count;
    int64_t first[sqk::kMaxBatch + 1];
    const int8_t* w[sqk::kMaxBatch];
    const void* s[sqk::kMaxBatch];  // fp32, or binary16 (H)
    int8_t* wq[sqk::kMaxBatch];
    void* w_scale[sqk::kMaxBatch];  // fp32, or binary16 (H)
    int64_t n[sqk::kMaxBatch], kvec[sqk::kMaxBatch];
};

// element i of a scale array stored in fp32, or in binary16 (H)
template <bool H>
__device__ __forceinline__ float scale_at(const void* p, int64_t i) {
    if constexpr (H)
        return sqd::f16_dec(((const uint16_t*)p)[i]);
    else
        return ((const float*)p)[i];
}

// The row scale of a row whose max |W'| is m (floored), and the reciprocal
// the codes use. H: the scale is stored as binary16 and the reciprocal is
// that of the stored value (ADR-010 "Consequences"); the returned bits are
// the binary16 pattern, otherwise the fp32 pattern.
template <bool H>
__device__ __forceinline__ uint32_t row_scale(float m, float qmax, float& inv) {
    const float ws = __fdiv_rn(m, qmax);
    if constexpr (H) {
        const uint16_t h = sqd::scale_f16(ws);
        inv = sqd::f16_inv(h);
        return h;
    } else {
        inv = __fdiv_rn(1.0f, ws);
        return __float_as_uint(ws);
    }
}

template <bool H>
__device__ __forceinline__ void store_scale(void* p, int64_t i, uint32_t bits) {
    if constexpr (H)
        ((uint16_t*)p)[i] = (uint16_t)bits;
    else
        ((float*)p)[i] = __uint_as_float(bits);
}

__device__ __forceinline__ int stage_item(const QwTable& tab, int64_t g) {
    int i = 0;
    while (i + 1 < tab.count && g >= tab.first[i + 1]) ++i;
    return i;
}

template <int EB, int WV, int NV, int RB, int CPW, int NS, bool FP8, bool H>
__global__ __launch_bounds__(64 * WV) void quant_weight_stream_kernel(const QwTable tab) {
    static_assert(!(FP8 && H), "binary16 scales are for int8 codes");
    constexpr int T = 64 * WV;                 // threads
    constexpr int E = 16 / EB;                 // elements per 16-byte vector
    constexpr int STAGE = CPW * WV * 1024;     // bytes, >= RB rows (checked by the launcher)
    constexpr int W32 = E / 4;                 // dwords of codes per vector
    static_assert(NS == 2 || NS == 3, "ring depth");
    static_assert((NS - 1) * CPW < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char ring[NS * STAGE];
    __shared__ float part[RB][WV];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t nstages = tab.first[tab.count];

    // this thread's slots for the current weight: vector j = t + i T of a
    // stage (live when j < RB * kvec), its row and its s values
    float sv[NV][E];
    int row[NV];
    bool live[NV];
    int cur = -1;
    auto setup = [&](int it) {
        const int kvec = (int)tab.kvec[it];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = t + i * T;
            live[i] = j < RB * kvec;
            row[i] = live[i] ? j / kvec : RB;
            const int c = live[i] ? j - row[i] * kvec : 0;
#pragma unroll
            for (int e = 0; e < E; ++e) sv[i][e] = live[i] ? scale_at<H>(tab.s[it], c * E + e) : 0.0f;
        }
        cur = it;
    };

    // stage g -> ring slot: CPW loads per wave, chunk c = wave + WV j of the
    // stage's contiguous bytes (zeros past the last row of its weight, and for
    // stages past the end)
    auto issue = [&](int64_t g, int slot) {
        const bool in = g < nstages;
        const int it = in ? stage_item(tab, g) : 0;
        const int64_t rowbytes = tab.kvec[it] * 16;
        const int64_t r0 = in ? (g - tab.first[it]) * RB : 0;
        const int64_t rows = in ? min<int64_t>(RB, tab.n[it] - r0) : 0;
        const sqd::i32x4 rsrc = sqd::tile_rsrc(tab.w[it] + r0 * rowbytes, rows, rowbytes);
        const uint32_t base = sqd::lds_addr(ring) + (uint32_t)(slot * STAGE) + (uint32_t)wave * 1024u;
#pragma unroll
        for (int j = 0; j < CPW; ++j)
            sqd::dma16(rsrc, base + (uint32_t)(j * WV * 1024), lane * 16, (j * WV + wave) * 1024);
    };

    // Codes of a stage are stored one round late (after the next stage's
    // wait), so the wait below, which also counts stores, finds them long
    // done; it is exact for the loads because loads complete in order and
    // exactly NS - 2 stages of loads are issued after the awaited one (the s
    // reloads at an item change only add younger operations, which makes the
    // wait stricter, never looser).
    uint32_t codes[NV][W32];
    uint32_t scale[RB];  // bit patterns (fp32, or binary16 when H)
    int64_t prev = -1;  // stage whose codes are pending
    auto flush = [&]() {
        if (prev < 0) return;
        const int64_t kvec = tab.kvec[cur], n = tab.n[cur];
        const int64_t p0 = (prev - tab.first[cur]) * RB;
        int8_t* dst = tab.wq[cur] + p0 * kvec * E;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (live[i] && p0 + row[i] < n) {
                const int64_t j = t + (int64_t)i * T;
                if constexpr (W32 == 2)
                    *(sqd::u32x2*)(dst + j * E) = sqd::u32x2{codes[i][0], codes[i][1]};
                else
                    *(uint32_t*)(dst + j * E) = codes[i][0];
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r)
            if (t == r && p0 + r < n) store_scale<H>(tab.w_scale[cur], p0 + r, scale[r]);
    };

    int64_t g = blockIdx.x;
    int slot = 0;
    if (g < nstages) setup(stage_item(tab, g));
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) issue(g + (int64_t)p * gridDim.x, p);
    for (; g < nstages; g += gridDim.x) {
        sqd::wait_vmcnt<(NS - 2) * CPW>();  // this stage landed (for this wave's loads) ...
        __syncthreads();                    // ... and for every wave; the slot read last round is free
        const int it = stage_item(tab, g);
        flush();  // the previous stage's codes (its weight is still `cur`)
        issue(g + (int64_t)(NS - 1) * gridDim.x, (slot + NS - 1) % NS);
        if (it != cur) setup(it);
        const char* st = ring + slot * STAGE;
        float wv[NV][E];
        float mx[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) mx[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float vm = 0.0f;
            if (live[i]) {
                const u32x4 raw = *(const u32x4*)(st + (t + i * T) * 16);
                float e[E];
                sqd::unpack16<E>(raw, e);
#pragma unroll
                for (int q = 0; q < E; ++q) {
                    wv[i][q] = __fmul_rn(e[q], sv[i][q]);
                    vm = __builtin_fmaxf(vm, __builtin_fabsf(wv[i][q]));
                }
            } else {
#pragma unroll
                for (int q = 0; q < E; ++q) wv[i][q] = 0.0f;
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) mx[r] = row[i] == r ? __builtin_fmaxf(mx[r], vm) : mx[r];
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            mx[r] = sqd::wave_max(mx[r]);
            if (lane == 0) part[r][wave] = mx[r];
        }
        __syncthreads();
        float inv[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            float m = part[r][0];
#pragma unroll
            for (int w = 1; w < WV; ++w) m = __builtin_fmaxf(m, part[r][w]);
            m = __builtin_fmaxf(m, sqd::kFloor);
            scale[r] = row_scale<H>(m, FP8 ? sqd::kFp8Max : sqd::kQmax, inv[r]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float inv_ws = inv[0];
#pragma unroll
            for (int r = 1; r < RB; ++r) inv_ws = row[i] == r ? inv[r] : inv_ws;
            if constexpr (FP8) {
                // e4m3 codes: |W' / ws| <= 448 (1 + 3 * 2^-24), which rounds to 448
#pragma unroll
                for (int d = 0; d < W32; ++d)
                    codes[i][d] = sqd::pack4_e4m3(
                        __fmul_rn(wv[i][4 * d], inv_ws), __fmul_rn(wv[i][4 * d + 1], inv_ws),
                        __fmul_rn(wv[i][4 * d + 2], inv_ws), __fmul_rn(wv[i][4 * d + 3], inv_ws));
            } else {
                // Codes by the round-to-nearest-even of the fp32 adder: for
                // |v| < 2^22, fl(v + 1.5 * 2^23) = rint(v) + 1.5 * 2^23 exactly,
                // and the low byte of its bit pattern is rint(v) as a
                // two's-complement int8. No clamp is needed: |W'| <= m and
                // inv_ws = fl(1 / fl(m / 127)), so |v| <= 127 (1 + 3 * 2^-24) and
                // rint(v) is within [-127, 127] (below the 1e-5 floor, |v| < 127).
                // Equal to q8() for every value this row can produce. A
                // binary16 row scale can sit below the fp32 one (by 2^-11
                // relative, far more where it is subnormal), so H clamps
                // first (rint and the integer clamp commute).
                uint32_t b[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float v = __fmul_rn(wv[i][e], inv_ws);
                    if constexpr (H) v = __builtin_fminf(__builtin_fmaxf(v, -sqd::kQmax), sqd::kQmax);
                    b[e] = __float_as_uint(__fadd_rn(v, 12582912.0f));
                }
#pragma unroll
                for (int d = 0; d < W32; ++d) {
                    // low bytes of b[4d .. 4d+3] -> one dword
                    const uint32_t lo = __builtin_amdgcn_perm(b[4 * d + 1], b[4 * d], 0x0c0c0400u);
                    const uint32_t hi = __builtin_amdgcn_perm(b[4 * d + 3], b[4 * d + 2], 0x0c0c0400u);
                    codes[i][d] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
            }
        }
        prev = g;
        slot = (slot + 1) % NS;
    }
    flush();
    sqd::wait_vmcnt<0>();  // zero-fill loads past the end may still be in flight
}

// Rows longer than 4096 groups (k > 65536): one block per row, the row is
// read twice and s is read from cache.
template <int EB, bool FP8, bool H>
__global__ __launch_bounds__(256) void quant_weight_long_kernel(const u32x4* __restrict__ w, int64_t kgroups,
                                                                const void* __restrict__ s,
                                                                int8_t* __restrict__ wq, void* __restrict__ w_scale) {
    static_assert(!(FP8 && H), "binary16 scales are for int8 codes");
    constexpr int VG = Group<EB>::V;
    auto load_s = [&](int64_t gi, float (&sv)[16]) {
        if constexpr (H) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const u32x4 t = ((const u32x4*)((const uint16_t*)s + gi * 16))[q];
                const uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sv[8 * q + 2 * u] = sqd::f16_dec((uint16_t)(d[u] & 0xffffu));
                    sv[8 * q + 2 * u + 1] = sqd::f16_dec((uint16_t)(d[u] >> 16));
                }
            }
        } else {
            load16f((const float*)s + gi * 16, sv);
        }
    };
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    float mx = 0.0f;
    for (int64_t gi = threadIdx.x; gi < kgroups; gi += 256) {
        Group<EB> raw;
        float e[16], sv[16];
        raw.load(w + (row * kgroups + gi) * VG);
        raw.widen(e);
        load_s(gi, sv);
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(__fmul_rn(e[j], sv[j])));
    }
    mx = __builtin_fmaxf(sqd::block_max<4>(mx, red), sqd::kFloor);
    float inv_ws;
    const uint32_t ws = row_scale<H>(mx, FP8 ? sqd::kFp8Max : sqd::kQmax, inv_ws);
    for (int64_t gi = threadIdx.x; gi < kgroups; gi += 256) {
        Group<EB> raw;
        float e[16], sv[16];
        int q[16];
        raw.load(w + (row * kgroups + gi) * VG);
        raw.widen(e);
        load_s(gi, sv);
        if constexpr (FP8) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = __fmul_rn(__fmul_rn(e[j], sv[j]), inv_ws);
            *(u32x4*)(wq + (row * kgroups + gi) * 16) =
                u32x4{sqd::pack4_e4m3(v[0], v[1], v[2], v[3]), sqd::pack4_e4m3(v[4], v[5], v[6], v[7]),
                      sqd::pack4_e4m3(v[8], v[9], v[10], v[11]), sqd::pack4_e4m3(v[12], v[13], v[14], v[15])};
            continue;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) q[j] = sqd::q8(__fmul_rn(__fmul_rn(e[j], sv[j]), inv_ws));
        store16(wq + (row * kgroups + gi) * 16, q);
    }
    if (threadIdx.x == 0) store_scale<H>(w_scale, row, ws);
}

constexpr int kActThreads = 256;
constexpr int kActUnroll = 8;
constexpr int kActShare = 4;  // consumers of one input quantized in one pass
// Rows per block: one round of kActUnroll loads per wave. Measured on MI355X
// against taller blocks (64-352 rows, each wave looping over rounds): 32-row
// blocks are as fast or faster on every shape, by 13-15 % at 65536 x 8192 and
// 262144 x 5120, where tall blocks leave a coarse last round of blocks.
constexpr int kActRowsPerBlock = 4 * kActUnroll;

// Activation inputs of several projections in one launch. Group g is one
// input x[rows, kvec vectors], read once; its consumers c = cfirst[g] ..
// cfirst[g + 1] - 1 (the projections fed by that input: q, k and v, or gate
// and up) each get their codes with their own inv_s and act_scale. Group g
// owns the blocks [first[g], first[g + 1]), strip-fastest.
struct ActTable {
    int count;
    int32_t first[sqk::kMaxBatch + 1];
    int32_t cfirst[sqk::kMaxBatch + 1];
    const u32x4* x[sqk::kMaxBatch];
    int64_t rows[sqk::kMaxBatch], kvec[sqk::kMaxBatch], rpb[sqk::kMaxBatch];
    int32_t strips[sqk::kMaxBatch], eb[sqk::kMaxBatch];
    const void* inv_s[sqk::kMaxBatch];      // fp32 inv_s, or the binary16 s (H)
    const void* act_scale[sqk::kMaxBatch];  // fp32, or binary16 (H)
    int8_t* xq[sqk::kMaxBatch];
};

// A lane owns one 16-byte column vector (E = 16 / EB elements) of the input
// and keeps the E inv_s values of each consumer in registers; the four waves
// of a block walk interleaved rows, so each wave instruction moves one
// contiguous 1 KB run.
//
// H: the scales are stored as binary16 (ADR-010 "Consequences"): inv_s[c]
// holds s itself and the lane forms fl(1 / s) of its columns once, and
// act_scale[c] is binary16; the arithmetic per element is unchanged.
template <int EB, bool FP8, int NC, bool O32 = false, bool H = false>
__device__ __forceinline__ void quant_act_block(const u32x4* __restrict__ x, int64_t rows, int64_t kvec,
                                                int64_t rows_per_block, int nc, const void* const (&inv_s)[NC],
                                                const void* const (&act_scale)[NC], int8_t* const (&xq)[NC],
                                                int64_t strip, int64_t chunk) {
    static_assert(!(FP8 && H), "binary16 scales are for int8 codes");
    constexpr int E = 16 / EB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t v = strip * 64 + lane;
    if (v >= kvec) return;  // no block-level synchronisation below
    float is[NC][E];
    float inv_a[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c >= nc) break;
        if constexpr (H) {
            // E binary16 values: 16 bytes (E = 8) or 8 bytes (E = 4)
            const uint16_t* sp = (const uint16_t*)inv_s[c] + v * E;
            uint32_t d[E / 2];
            if constexpr (E == 8) {
                const u32x4 t = *(const u32x4*)sp;
                d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
            } else {
                const sqd::u32x2 t = *(const sqd::u32x2*)sp;
                d[0] = t.x; d[1] = t.y;
            }
#pragma unroll
            for (int u = 0; u < E / 2; ++u) {
                is[c][2 * u] = sqd::f16_inv((uint16_t)(d[u] & 0xffffu));
                is[c][2 * u + 1] = sqd::f16_inv((uint16_t)(d[u] >> 16));
            }
            inv_a[c] = sqd::f16_inv(*(const uint16_t*)act_scale[c]);
        } else {
#pragma unroll
            for (int h = 0; h < E / 4; ++h) {
                const u32x4 t = ((const u32x4*)((const float*)inv_s[c] + v * E))[h];
                is[c][4 * h + 0] = __uint_as_float(t.x);
                is[c][4 * h + 1] = __uint_as_float(t.y);
                is[c][4 * h + 2] = __uint_as_float(t.z);
                is[c][4 * h + 3] = __uint_as_float(t.w);
            }
            inv_a[c] = __fdiv_rn(1.0f, *(const float*)act_scale[c]);
        }
    }
    const int64_t r0 = chunk * rows_per_block;
    const int64_t r1 = min(rows, r0 + rows_per_block);
    // global address space: pointers taken from a table are generic, and
    // generic (flat) accesses wait on both counters and cannot take a scalar base
    typedef __attribute__((address_space(1))) const u32x4 gvec;
    typedef __attribute__((address_space(1))) const char gcbyte;
    typedef __attribute__((address_space(1))) int8_t gbyte;
    gvec* gx = (gvec*)x;
    // O32: every tensor of the launch is below 4 GiB, so byte offsets fit 32
    // bits and an access is a scalar base plus one 32-bit offset, shared by
    // the consumers of a row
    using Off = typename std::conditional<O32, uint32_t, int64_t>::type;
    auto load = [&](int64_t r) -> u32x4 {
        const Off vec = (Off)r * (Off)kvec + (Off)v;
        return __builtin_nontemporal_load((gvec*)((gcbyte*)gx + vec * (Off)16));
    };
    auto quantize = [&](const u32x4& raw, int64_t r) {
        float e[E];
        sqd::unpack16<E>(raw, e);
        const Off off = ((Off)r * (Off)kvec + (Off)v) * (Off)E;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c >= nc) break;
            gbyte* dst = (gbyte*)xq[c] + off;
            if constexpr (FP8) {
                float t[E];
#pragma unroll
                for (int u = 0; u < E; ++u) t[u] = __fmul_rn(__fmul_rn(e[u], is[c][u]), inv_a[c]);
                if constexpr (E == 8)
                    *(__attribute__((address_space(1))) sqd::u32x2*)dst =
                        sqd::u32x2{sqd::pack4_e4m3(t[0], t[1], t[2], t[3]), sqd::pack4_e4m3(t[4], t[5], t[6], t[7])};
                else
                    *(__attribute__((address_space(1))) uint32_t*)dst = sqd::pack4_e4m3(t[0], t[1], t[2], t[3]);
            } else {
                // clamp to [-127, 127], then round half to even with the fp32
                // adder (fl(v + 1.5 * 2^23) keeps rint(v) in its low byte for
                // |v| < 2^22; rint and the integer-bounded clamp commute, so
                // this is clamp(rint(v))), and gather the low bytes with v_perm
                uint32_t b[E];
#pragma unroll
                for (int t = 0; t < E; ++t) {
                    const float q = __builtin_fminf(
                        __builtin_fmaxf(__fmul_rn(__fmul_rn(e[t], is[c][t]), inv_a[c]), -sqd::kQmax), sqd::kQmax);
                    b[t] = __float_as_uint(__fadd_rn(q, 12582912.0f));
                }
                uint32_t w[E / 4];
#pragma unroll
                for (int d = 0; d < E / 4; ++d) {
                    const uint32_t lo = __builtin_amdgcn_perm(b[4 * d + 1], b[4 * d], 0x0c0c0400u);
                    const uint32_t hi = __builtin_amdgcn_perm(b[4 * d + 3], b[4 * d + 2], 0x0c0c0400u);
                    w[d] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
                if constexpr (E == 8)
                    *(__attribute__((address_space(1))) sqd::u32x2*)dst = sqd::u32x2{w[0], w[1]};
                else
                    *(__attribute__((address_space(1))) uint32_t*)dst = w[0];
            }
        }
    };
    int64_t r = r0 + wave;
    for (; r + 4 * (kActUnroll - 1) < r1; r += 4 * kActUnroll) {
        u32x4 t[kActUnroll];
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) t[u] = load(r + 4 * u);
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) quantize(t[u], r + 4 * u);
    }
    for (; r < r1; r += 4) quantize(load(r), r);
}

// one input, one consumer, arguments in kernel parameters: the single-call form
template <int EB, bool FP8, bool H>
__global__ __launch_bounds__(kActThreads) void quant_act_kernel(const u32x4* __restrict__ x, int64_t rows,
                                                                int64_t kvec, int64_t rows_per_block,
                                                                const void* __restrict__ inv_s,
                                                                const void* __restrict__ act_scale,
                                                                int8_t* __restrict__ xq) {
    const void* is[1] = {inv_s};
    const void* as[1] = {act_scale};
    int8_t* q[1] = {xq};
    quant_act_block<EB, FP8, 1, false, H>(x, rows, kvec, rows_per_block, 1, is, as, q, blockIdx.x, blockIdx.y);
}

// NC: the most consumers any group of the launch has (1, 2 or 4): a group's
// inv_s registers scale with it, and a single consumer keeps the occupancy of
// a plain quantizer
template <int EB, bool FP8, int NC, bool O32, bool H>
__global__ __launch_bounds__(kActThreads) void quant_act_batched_kernel(const ActTable tab) {
    // the group's fields as plain scalars: the block then addresses its
    // input and outputs exactly as a kernel taking them as arguments would
    const int g = sqd::item_of(tab.first, tab.count, blockIdx.x);
    const int32_t local = blockIdx.x - tab.first[g], strips = tab.strips[g];
    const int cf = tab.cfirst[g], nc = tab.cfirst[g + 1] - cf;
    const void* inv_s[NC];
    const void* act_scale[NC];
    int8_t* xq[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int ci = c < nc ? cf + c : cf;
        inv_s[c] = tab.inv_s[ci];
        act_scale[c] = tab.act_scale[ci];
        xq[c] = tab.xq[ci];
    }
    const u32x4* x = tab.x[g];
    const int64_t rows = tab.rows[g], kvec = tab.kvec[g], rpb = tab.rpb[g];
    // integer division has no scalar instruction: bring the block-uniform
    // quotient back to a scalar register so everything derived from it is too
    const int32_t chunk = __builtin_amdgcn_readfirstlane(local / strips), strip = local - chunk * strips;
    quant_act_block<EB, FP8, NC, O32, H>(x, rows, kvec, rpb, nc, inv_s, act_scale, xq, strip, chunk);
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

// WV waves of 64 threads, NV vector slots per thread, RB rows per stage of
// CPW KB per wave, NS stages in the ring, PER_CU blocks per compute unit (the
// rings of all of them fit the LDS)
template <int EB, int WV, int NV, int RB, int CPW, int NS, int PER_CU, bool FP8, bool H>
hipError_t launch_qw(const QwTable& tab, hipStream_t stream) {
    static_assert(PER_CU * (NS * CPW * WV * 1024 + RB * WV * 4) <= 160 * 1024, "the rings fit in LDS");
    for (int i = 0; i < tab.count; ++i)
        if (RB * tab.kvec[i] * 16 > CPW * WV * 1024 || RB * tab.kvec[i] > NV * 64 * WV) return hipErrorInvalidValue;
    const int64_t blocks = std::min<int64_t>(tab.first[tab.count], (int64_t)PER_CU * device_cus());
    quant_weight_stream_kernel<EB, WV, NV, RB, CPW, NS, FP8, H><<<dim3((unsigned)blocks), dim3(64 * WV), 0, stream>>>(
        tab);
    return hipGetLastError();
}

// Kernel shape for rows of kvec 16-byte vectors (waves, slots per thread,
// rows per stage, KB per wave per stage, ring depth, blocks per compute unit),
// measured on MI355X over the Llama-2 7B/13B/70B projections: stages of
// 16-64 KB in a two-deep ring and two to four blocks per compute unit, so that
// while one block reduces and quantizes a stage the others' loads keep HBM
// busy; the slots per thread divide a stage's vectors (nearly) evenly.
// Shape 8: rows of more than 4096 vectors, one block per row reading it twice.
constexpr int kQwLong = 8;
constexpr int kQwRowsPerStage[kQwLong] = {4, 2, 2, 2, 1, 1, 1, 1};

int qw_shape(int64_t kvec) {
    if (kvec <= 256) return 0;
    if (kvec <= 512) return 1;
    if (kvec <= 640) return 2;
    if (kvec <= 1024) return 3;
    if (kvec <= 1536) return 4;
    if (kvec <= 1792) return 5;
    if (kvec <= 2048) return 6;
    if (kvec <= 4096) return 7;
    return kQwLong;
}

template <int EB, bool FP8, bool H>
hipError_t launch_shape(int shape, const QwTable& tab, hipStream_t stream) {
    switch (shape) {
        case 0: return launch_qw<EB, 4, 4, 4, 4, 2, 4, FP8, H>(tab, stream);
        case 1: return launch_qw<EB, 4, 4, 2, 4, 2, 4, FP8, H>(tab, stream);
        case 2: return launch_qw<EB, 4, 5, 2, 5, 2, 3, FP8, H>(tab, stream);
        case 3: return launch_qw<EB, 8, 4, 2, 4, 2, 2, FP8, H>(tab, stream);
        case 4: return launch_qw<EB, 8, 3, 1, 3, 2, 3, FP8, H>(tab, stream);
        case 5: return launch_qw<EB, 4, 7, 1, 7, 2, 2, FP8, H>(tab, stream);
        case 6: return launch_qw<EB, 8, 4, 1, 4, 2, 2, FP8, H>(tab, stream);
        case 7: return launch_qw<EB, 16, 4, 1, 4, 2, 1, FP8, H>(tab, stream);
    }
    return hipErrorInvalidValue;
}

// Items of one element type, scale storage and kernel shape share a launch
// (first-appearance order); long rows get a launch per item.
template <bool FP8, bool H>
hipError_t quant_weight_items(const sqk::QuantWeightItem* items, int count, hipStream_t stream) {
    bool done[sqk::kMaxBatch] = {};
    for (int i = 0; i < count; ++i) {
        if (done[i] || items[i].h != H) continue;
        done[i] = true;
        if (items[i].n == 0) continue;
        const int eb = sqk::elem_bytes(items[i].wt);
        const int shape = qw_shape(items[i].k * eb / 16);
        if (shape == kQwLong) {
            const int64_t kgroups = items[i].k / 16;
            if (eb == 2)
                quant_weight_long_kernel<2, FP8, H><<<dim3((unsigned)items[i].n), dim3(256), 0, stream>>>(
                    (const u32x4*)items[i].w, kgroups, items[i].s, items[i].wq, items[i].w_scale);
            else
                quant_weight_long_kernel<4, FP8, H><<<dim3((unsigned)items[i].n), dim3(256), 0, stream>>>(
                    (const u32x4*)items[i].w, kgroups, items[i].s, items[i].wq, items[i].w_scale);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            continue;
        }
        QwTable tab{};
        int64_t stages = 0;
        for (int j = i; j < count; ++j) {
            if (j > i && (done[j] || items[j].n == 0 || items[j].h != H || sqk::elem_bytes(items[j].wt) != eb ||
                          qw_shape(items[j].k * eb / 16) != shape))
                continue;
            done[j] = true;
            const int c = tab.count++;
            tab.first[c] = stages;
            tab.w[c] = (const int8_t*)items[j].w;
            tab.s[c] = items[j].s;
            tab.wq[c] = items[j].wq;
            tab.w_scale[c] = items[j].w_scale;
            tab.n[c] = items[j].n;
            tab.kvec[c] = items[j].k * eb / 16;
            stages += (items[j].n + kQwRowsPerStage[shape] - 1) / kQwRowsPerStage[shape];
        }
        tab.first[tab.count] = stages;
        const hipError_t e =
            eb == 2 ? launch_shape<2, FP8, H>(shape, tab, stream) : launch_shape<4, FP8, H>(shape, tab, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

namespace sqk {

hipError_t quant_weight(const void* w, int wt, int64_t n, int64_t k, const void* s, int8_t* wq,
                        void* w_scale, bool h, hipStream_t stream) {
    const QuantWeightItem item{w, wt, n, k, s, wq, w_scale, h};
    return quant_weight_batched(&item, 1, stream);
}

hipError_t quant_weight_batched(const QuantWeightItem* items, int count, hipStream_t stream) {
    const hipError_t e = quant_weight_items<false, false>(items, count, stream);
    return e != hipSuccess ? e : quant_weight_items<false, true>(items, count, stream);
}

hipError_t quant_weight_fp8_batched(const QuantWeightItem* items, int count, hipStream_t stream) {
    for (int i = 0; i < count; ++i)
        if (items[i].h) return hipErrorInvalidValue;
    return quant_weight_items<true, false>(items, count, stream);
}

hipError_t quant_weight_fp8(const void* w, int wt, int64_t n, int64_t k, const float* s, uint8_t* wq,
                            float* w_scale, hipStream_t stream) {
    const QuantWeightItem item{w, wt, n, k, s, (int8_t*)wq, w_scale, false};
    return quant_weight_items<true, false>(&item, 1, stream);
}

template <int EB, bool FP8, int NC, bool H>
void launch_act(const ActTable& tab, int64_t blocks, bool o32, hipStream_t stream) {
    if (o32)
        quant_act_batched_kernel<EB, FP8, NC, true, H><<<dim3((unsigned)blocks), dim3(kActThreads), 0, stream>>>(tab);
    else
        quant_act_batched_kernel<EB, FP8, NC, false, H><<<dim3((unsigned)blocks), dim3(kActThreads), 0, stream>>>(
            tab);
}

// Items with the same input (pointer, type and shape) form one group, up to
// kActShare consumers each, in first-appearance order; one launch per element
// type among the inputs. H: only the items with binary16 scales (the others
// only those without).
template <bool FP8, bool H>
hipError_t quant_act_items(const ActItem* items, int count, hipStream_t stream) {
    bool done[kMaxBatch] = {};
    for (int i = 0; i < count; ++i) done[i] = items[i].h != H;
    for (int eb : {2, 4}) {
        ActTable tab{};
        int ng = 0, nc = 0, widest = 1;
        int64_t blocks = 0;
        bool o32 = true;  // every input (and so every code tensor) below 4 GiB
        for (int i = 0; i < count; ++i) {
            if (done[i] || items[i].m == 0 || elem_bytes(items[i].xt) != eb) continue;
            const int64_t kvec = items[i].k * eb / 16;
            const int64_t strips = (kvec + 63) / 64;
            const int64_t rpb = kActRowsPerBlock;
            const int64_t chunks = (items[i].m + rpb - 1) / rpb;
            tab.first[ng] = (int32_t)blocks;
            tab.cfirst[ng] = nc;
            tab.x[ng] = (const u32x4*)items[i].x;
            tab.rows[ng] = items[i].m;
            tab.kvec[ng] = kvec;
            tab.rpb[ng] = rpb;
            tab.strips[ng] = (int32_t)strips;
            tab.eb[ng] = eb;
            o32 = o32 && items[i].m * kvec * 16 < ((int64_t)1 << 32);
            int shared = 0;
            for (int j = i; j < count && shared < kActShare; ++j) {
                if (done[j] || items[j].x != items[i].x || items[j].xt != items[i].xt || items[j].m != items[i].m ||
                    items[j].k != items[i].k)
                    continue;
                done[j] = true;
                tab.inv_s[nc] = items[j].inv_s;
                tab.act_scale[nc] = items[j].act_scale;
                tab.xq[nc] = items[j].xq;
                ++nc;
                ++shared;
            }
            blocks += strips * chunks;
            widest = std::max(widest, shared);
            ++ng;  // consumers of this input beyond kActShare start a group of their own further on
        }
        if (ng == 0) continue;
        if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        tab.count = ng;
        tab.first[ng] = (int32_t)blocks;
        tab.cfirst[ng] = nc;
        if (eb == 2) {
            if (widest == 1) launch_act<2, FP8, 1, H>(tab, blocks, o32, stream);
            else if (widest == 2) launch_act<2, FP8, 2, H>(tab, blocks, o32, stream);
            else launch_act<2, FP8, kActShare, H>(tab, blocks, o32, stream);
        } else {
            if (widest == 1) launch_act<4, FP8, 1, H>(tab, blocks, o32, stream);
            else if (widest == 2) launch_act<4, FP8, 2, H>(tab, blocks, o32, stream);
            else launch_act<4, FP8, kActShare, H>(tab, blocks, o32, stream);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// one input and one consumer: the kernel with plain arguments (no table to
// look the group up in), blocks of 4 waves over 32 rows of a 64-vector strip
template <bool FP8, bool H>
hipError_t quant_act_single(const void* x, int xt, int64_t m, int64_t k, const void* inv_s,
                            const void* act_scale, int8_t* xq, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    const int eb = elem_bytes(xt);
    const int64_t kvec = k * eb / 16;
    const int64_t strips = (kvec + 63) / 64;
    int64_t rpb = kActRowsPerBlock;
    int64_t chunks = (m + rpb - 1) / rpb;
    if (chunks > 65535) {  // the grid's second dimension: taller blocks, still whole rounds of loads
        rpb = (m + 65534) / 65535;
        rpb = (rpb + kActRowsPerBlock - 1) / kActRowsPerBlock * kActRowsPerBlock;
        chunks = (m + rpb - 1) / rpb;
    }
    const dim3 grid((unsigned)strips, (unsigned)chunks), block(kActThreads);
    if (eb == 2)
        quant_act_kernel<2, FP8, H><<<grid, block, 0, stream>>>((const u32x4*)x, m, kvec, rpb, inv_s, act_scale, xq);
    else
        quant_act_kernel<4, FP8, H><<<grid, block, 0, stream>>>((const u32x4*)x, m, kvec, rpb, inv_s, act_scale, xq);
    return hipGetLastError();
}

hipError_t quant_act(const void* x, int xt, int64_t m, int64_t k, const void* inv_s, const void* act_scale,
                     int8_t* xq, bool h, hipStream_t stream) {
    return h ? quant_act_single<false, true>(x, xt, m, k, inv_s, act_scale, xq, stream)
             : quant_act_single<false, false>(x, xt, m, k, inv_s, act_scale, xq, stream);
}

hipError_t quant_act_batched(const ActItem* items, int count, hipStream_t stream) {
    const hipError_t e = quant_act_items<false, false>(items, count, stream);
    return e != hipSuccess ? e : quant_act_items<false, true>(items, count, stream);
}

hipError_t quant_act_fp8_batched(const ActItem* items, int count, hipStream_t stream) {
    for (int i = 0; i < count; ++i)
        if (items[i].h) return hipErrorInvalidValue;
    return quant_act_items<true, false>(items, count, stream);
}

hipError_t quant_act_fp8(const void* x, int xt, int64_t m, int64_t k, const float* inv_s, const float* act_scale,
                         uint8_t* xq, hipStream_t stream) {
    return quant_act_single<true, false>(x, xt, m, k, inv_s, act_scale, (int8_t*)xq, stream);
}

}  // namespace sqk
