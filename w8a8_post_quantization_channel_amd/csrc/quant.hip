// quant.hip -- the two quantization passes of the SmoothQuant W8A8 layer.
//
// quant_weight: offline fold W' = W diag(s) (kwkr.cn blog §3.2) and symmetric
//   int8 with one scale per output row (ADR-010 "Context" item 3). A block
//   owns whole rows: its threads load every vector of them at once, keep W'
//   in registers between the row max and the quantize pass, and store the
//   codes with streaming stores, so W is read from HBM exactly once.
// quant_act: runtime x * (1/s) strictly before the per-tensor quantizer
//   (kwkr.cn blog §3.2 and §5.2; ADR-010 "Key design" items 4-5). A lane owns
//   one 16-byte column vector and keeps its inv_s values in registers while
//   the four waves of a block walk interleaved rows.
//
// The pass for rows longer than 4096 vectors works on "groups" of 16
// consecutive elements of a row (32 bytes of bf16, 64 of fp32), which become
// 16 int8 codes: one 16-byte store.
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

// Weight rows as whole-row blocks. A block of T = 64 WV threads (WV <= 16,
// chosen per weight so that NV * T just covers a row of kvec 16-byte vectors)
// quantizes RPB consecutive rows. Thread t owns the vectors t, t + T, ... (NV
// of them) of each of the rows and issues all RPB * NV loads at once; it
// loads the s values of its columns once for the RPB rows, forms W' = W * s in
// registers, and the row maxima come from wave reductions and one LDS
// exchange. The codes then go out with streaming stores (the codes of a
// weight are read back only by later GEMMs). W is read from HBM once.
//
// No block is persistent: a compute unit holds several blocks at a time and
// starts the next one as one retires, which keeps more of W in flight than a
// persistent block ring: measured on MI355X over the Llama-2 projections, the
// whole-row blocks are 10-25 % faster than an LDS ring of prefetched stages.
//
// One launch can cover several weights of equal block size (the projections
// of a block): item i owns the blocks [first[i], first[i + 1]).

struct QwTable {
    int count;
    int32_t first[sqk::kMaxBatch + 1];
    const u32x4* w[sqk::kMaxBatch];
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

// the E scale values of column vector c (E = 8: bf16 weights, E = 4: fp32)
template <int E, bool H>
__device__ __forceinline__ void load_scales(const void* __restrict__ s, int64_t c, float (&sv)[E]) {
    if constexpr (H) {
        uint32_t d[E / 2];
        if constexpr (E == 8) {
            const u32x4 t = ((const u32x4*)s)[c];
            d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
        } else {
            const sqd::u32x2 t = ((const sqd::u32x2*)s)[c];
            d[0] = t.x; d[1] = t.y;
        }
#pragma unroll
        for (int u = 0; u < E / 2; ++u) {
            sv[2 * u] = sqd::f16_dec((uint16_t)(d[u] & 0xffffu));
            sv[2 * u + 1] = sqd::f16_dec((uint16_t)(d[u] >> 16));
        }
    } else {
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
            const u32x4 t = ((const u32x4*)s)[c * (E / 4) + h];
            sv[4 * h + 0] = __uint_as_float(t.x);
            sv[4 * h + 1] = __uint_as_float(t.y);
            sv[4 * h + 2] = __uint_as_float(t.z);
            sv[4 * h + 3] = __uint_as_float(t.w);
        }
    }
}

template <int EB, int NV, int RPB, bool FP8, bool H>
__global__ __launch_bounds__(1024) void quant_weight_rows_kernel(const QwTable tab) {
    static_assert(!(FP8 && H), "binary16 scales are for int8 codes");
    constexpr int E = 16 / EB;    // elements per 16-byte vector
    constexpr int W32 = E / 4;    // dwords of codes per vector
    __shared__ float part[RPB][16];

    const int b = blockIdx.x;
    int it = 0;
    while (it + 1 < tab.count && b >= tab.first[it + 1]) ++it;
    const u32x4* __restrict__ w = tab.w[it];
    const int64_t n = tab.n[it], kvec = tab.kvec[it];
    const int64_t r0 = (int64_t)(b - tab.first[it]) * RPB;
    const int T = blockDim.x, WV = T >> 6;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    bool live[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) live[i] = t + i * T < kvec;
    u32x4 raw[RPB][NV];
#pragma unroll
    for (int p = 0; p < RPB; ++p)
#pragma unroll
        for (int i = 0; i < NV; ++i)
            raw[p][i] = live[i] && r0 + p < n ? __builtin_nontemporal_load(w + (r0 + p) * kvec + t + i * T)
                                              : u32x4{0, 0, 0, 0};
    float sv[NV][E];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (live[i]) {
            load_scales<E, H>(tab.s[it], t + i * T, sv[i]);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) sv[i][e] = 0.0f;
        }
    }

    // pass 1: W' = W * s in registers and the row maxima
    float wv[RPB][NV][E];
#pragma unroll
    for (int p = 0; p < RPB; ++p) {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float e8[E];
            sqd::unpack16<E>(raw[p][i], e8);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                wv[p][i][e] = __fmul_rn(e8[e], sv[i][e]);
                mx = __builtin_fmaxf(mx, __builtin_fabsf(wv[p][i][e]));
            }
        }
        mx = sqd::wave_max(mx);
        if (lane == 0) part[p][wave] = mx;
    }
    __syncthreads();

    // pass 2: the row scale and the codes
#pragma unroll
    for (int p = 0; p < RPB; ++p) {
        if (r0 + p >= n) break;
        float m = part[p][0];
        for (int q = 1; q < WV; ++q) m = __builtin_fmaxf(m, part[p][q]);
        m = __builtin_fmaxf(m, sqd::kFloor);
        float inv_ws;
        const uint32_t scale = row_scale<H>(m, FP8 ? sqd::kFp8Max : sqd::kQmax, inv_ws);
        int8_t* dst = tab.wq[it] + (r0 + p) * kvec * E;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (!live[i]) continue;
            uint32_t codes[W32];
            if constexpr (FP8) {
                // e4m3 codes: |W' / ws| <= 448 (1 + 3 * 2^-24), which rounds to 448
#pragma unroll
                for (int d = 0; d < W32; ++d)
                    codes[d] = sqd::pack4_e4m3(
                        __fmul_rn(wv[p][i][4 * d], inv_ws), __fmul_rn(wv[p][i][4 * d + 1], inv_ws),
                        __fmul_rn(wv[p][i][4 * d + 2], inv_ws), __fmul_rn(wv[p][i][4 * d + 3], inv_ws));
            } else {
                // Codes by the round-to-nearest-even of the fp32 adder: for
                // |v| < 2^22, fl(v + 1.5 * 2^23) = rint(v) + 1.5 * 2^23 exactly,
                // and the low byte of its bit pattern is rint(v) as a
                // two's-complement int8. No clamp is needed for fp32 scales:
                // |W'| <= m and inv_ws = fl(1 / fl(m / 127)), so
                // |v| <= 127 (1 + 3 * 2^-24) and rint(v) is within [-127, 127]
                // (below the 1e-5 floor, |v| < 127). A binary16 row scale can
                // sit below the fp32 one (by 2^-11 relative, far more where it
                // is subnormal), so H clamps first (rint and the integer clamp
                // commute). Equal to q8() for every value the row can produce.
                uint32_t bits[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float v = __fmul_rn(wv[p][i][e], inv_ws);
                    if constexpr (H) v = __builtin_fminf(__builtin_fmaxf(v, -sqd::kQmax), sqd::kQmax);
                    bits[e] = __float_as_uint(__fadd_rn(v, 12582912.0f));
                }
#pragma unroll
                for (int d = 0; d < W32; ++d) {
                    // low bytes of bits[4d .. 4d+3] -> one dword
                    const uint32_t lo = __builtin_amdgcn_perm(bits[4 * d + 1], bits[4 * d], 0x0c0c0400u);
                    const uint32_t hi = __builtin_amdgcn_perm(bits[4 * d + 3], bits[4 * d + 2], 0x0c0c0400u);
                    codes[d] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
            }
            int8_t* q = dst + (int64_t)(t + i * T) * E;
            if constexpr (W32 == 2)
                __builtin_nontemporal_store(sqd::u32x2{codes[0], codes[1]}, (sqd::u32x2*)q);
            else
                __builtin_nontemporal_store(codes[0], (uint32_t*)q);
        }
        if (t == 0) store_scale<H>(tab.w_scale[it], r0 + p, scale);
    }
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
    // The codes go out with ordinary stores: the GEMM that reads them next
    // finds them in the cache. Streaming stores made this pass alone 5 %
    // faster on 4096 x 28672 but the 13B layer step 0.8 % slower (its GEMM
    // 574 -> 582 us, same box), so they are kept for the weight codes only.
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

// Vector slots per thread and rows per block for rows of kvec 16-byte
// vectors: (2, 2) for rows of up to 1024 vectors (blocks of up to 512
// threads), (4, 1) up to 4096 (up to 1024 threads); longer rows take
// quant_weight_long_kernel. Measured on MI355X over Llama-2 7B/13B/70B
// projection shapes against 1-6 slots and 1-6 rows: these two are within a
// few percent of the best on every shape.
constexpr int64_t kQwShortRow = 1024, kQwMaxRow = 4096;

int qw_slots(int64_t kvec) { return kvec <= kQwShortRow ? 2 : 4; }
int qw_rows(int64_t kvec) { return kvec <= kQwShortRow ? 2 : 1; }
// threads per block: the multiple of 64 that NV slots each just cover
int qw_threads(int64_t kvec) {
    const int64_t nv = qw_slots(kvec);
    return (int)((kvec + nv - 1) / nv + 63) / 64 * 64;
}

template <int EB, int NV, int RPB, bool FP8, bool H>
void launch_rows(const QwTable& tab, int threads, hipStream_t stream) {
    quant_weight_rows_kernel<EB, NV, RPB, FP8, H><<<dim3((unsigned)tab.first[tab.count]), dim3(threads), 0, stream>>>(
        tab);
}

// Items of one element type and scale storage whose rows take the same block
// size share a launch (first-appearance order); long rows get a launch per
// item.
template <bool FP8, bool H>
hipError_t quant_weight_items(const sqk::QuantWeightItem* items, int count, hipStream_t stream) {
    bool done[sqk::kMaxBatch] = {};
    for (int i = 0; i < count; ++i) {
        if (done[i] || items[i].h != H) continue;
        done[i] = true;
        if (items[i].n == 0) continue;
        const int eb = sqk::elem_bytes(items[i].wt);
        const int64_t kvec = items[i].k * eb / 16;
        if (kvec > kQwMaxRow) {
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
        const int threads = qw_threads(kvec);
        const bool short_rows = kvec <= kQwShortRow;
        QwTable tab{};
        int64_t blocks = 0;
        for (int j = i; j < count; ++j) {
            if (j > i && (done[j] || items[j].n == 0 || items[j].h != H || sqk::elem_bytes(items[j].wt) != eb))
                continue;
            const int64_t kv = items[j].k * eb / 16;
            if (j > i && (kv > kQwMaxRow || (kv <= kQwShortRow) != short_rows || qw_threads(kv) != threads))
                continue;
            done[j] = true;
            const int c = tab.count++;
            tab.first[c] = (int32_t)blocks;
            tab.w[c] = (const u32x4*)items[j].w;
            tab.s[c] = items[j].s;
            tab.wq[c] = items[j].wq;
            tab.w_scale[c] = items[j].w_scale;
            tab.n[c] = items[j].n;
            tab.kvec[c] = kv;
            blocks += (items[j].n + qw_rows(kv) - 1) / qw_rows(kv);
            if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        }
        tab.first[tab.count] = (int32_t)blocks;
        if (eb == 2)
            short_rows ? launch_rows<2, 2, 2, FP8, H>(tab, threads, stream)
                       : launch_rows<2, 4, 1, FP8, H>(tab, threads, stream);
        else
            short_rows ? launch_rows<4, 2, 2, FP8, H>(tab, threads, stream)
                       : launch_rows<4, 4, 1, FP8, H>(tab, threads, stream);
        const hipError_t e = hipGetLastError();
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
