// sq_device.h -- device-side helpers shared by the libsq kernels (gfx950 only).
//
// Numerics follow the fixed fp32 op order of the SmoothQuant W8A8 path: every
// product is one IEEE fp32 multiply (__fmul_rn, no contraction), divisions are
// correctly rounded (__fdiv_rn), integer codes are round-half-to-even
// (v_rndne_f32) clamped to [-127, 127] (symmetric quantizer of the kwkr.cn
// blog §1.2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kFloor = 1e-5f;  // guard floor on statistics (tbr8.org example clamps s at 1e-5)
constexpr float kQmax = 127.0f;  // symmetric int8 range [-127, 127]

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// round-to-nearest-even fp32 -> bf16 bit pattern (NaN kept quiet); written
// as a select so it compiles without branches
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;
}

// two fp32 values -> packed bf16 pair (low half = lo), one v_cvt_pk_bf16_f32:
// round-to-nearest-even like f32_to_bf16_bits for every normal value, zero
// and infinity
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// symmetric int8 code of an already scaled value
__device__ __forceinline__ int q8(float v) {
    float r = __builtin_rintf(v);
    r = __builtin_fminf(__builtin_fmaxf(r, -kQmax), kQmax);
    return (int)r;
}

// IEEE binary16 scale storage (ADR-010 "Consequences": the per-row weight
// scale, the per-tensor activation scale and the smoothing factors kept in
// fp16). v_cvt_f16_f32 rounds to nearest even in the default rounding mode
// and yields binary16 subnormals (fp16 denormals are kept in the default
// float mode of gfx950 kernels); v_cvt_f32_f16 is exact. A stored scale is
// clamped into [2^-24, 65504] first, so it is never zero nor infinite.
constexpr float kF16Min = 0x1p-24f;
constexpr float kF16Max = 65504.0f;

__device__ __forceinline__ float f16_dec(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint16_t scale_f16(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)__builtin_fminf(__builtin_fmaxf(v, kF16Min), kF16Max));
}

// fl(1 / decoded stored scale): the reciprocal the quantizers multiply by
__device__ __forceinline__ float f16_inv(uint16_t h) { return __fdiv_rn(1.0f, f16_dec(h)); }

// OCP FP8 E4M3 (bias 7, largest finite 448): four fp32 values, clamped to
// [-448, 448], rounded to nearest even by v_cvt_pk_fp8_f32, one byte each
// (a in the low byte).
constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    auto cl = [](float v) { return __builtin_fminf(__builtin_fmaxf(v, -kFp8Max), kFp8Max); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// Widen one 16-byte vector to fp32: 8 bf16 or 4 fp32 values.
template <int E>
__device__ __forceinline__ void unpack16(const u32x4& v, float (&e)[E]);

template <>
__device__ __forceinline__ void unpack16<8>(const u32x4& v, float (&e)[8]) {
    e[0] = bf16_lo(v.x); e[1] = bf16_hi(v.x);
    e[2] = bf16_lo(v.y); e[3] = bf16_hi(v.y);
    e[4] = bf16_lo(v.z); e[5] = bf16_hi(v.z);
    e[6] = bf16_lo(v.w); e[7] = bf16_hi(v.w);
}

template <>
__device__ __forceinline__ void unpack16<4>(const u32x4& v, float (&e)[4]) {
    e[0] = __uint_as_float(v.x); e[1] = __uint_as_float(v.y);
    e[2] = __uint_as_float(v.z); e[3] = __uint_as_float(v.w);
}

// Wave-wide maximum of non-negative values (64 lanes, all active). Bit
// patterns of non-negative floats order like unsigned integers, so the max is
// an exact integer max: DPP within each 16-lane row (quad swaps, then row
// rotations by 4 and 8), then the four row maxima read into scalars.
__device__ __forceinline__ float wave_max(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp((int)u, (int)u, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x124, 0xF, 0xF, false));  // row_ror:4
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x128, 0xF, 0xF, false));  // row_ror:8
    const uint32_t r0 = __builtin_amdgcn_readlane(u, 0), r1 = __builtin_amdgcn_readlane(u, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(u, 32), r3 = __builtin_amdgcn_readlane(u, 48);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// Wave-wide sum of int32 values (64 lanes, all active): the same DPP pattern
// as wave_max with integer adds, which are exact in any order.
__device__ __forceinline__ int wave_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);  // row_ror:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
           __builtin_amdgcn_readlane(v, 48);
}

// block-wide maximum of non-negative values; every thread gets the result.
// `red` holds >= NWAVES floats.
template <int NWAVES>
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) r = __builtin_fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// ---- global -> LDS direct loads (buffer_load ... lds) --------------------------

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Raw buffer descriptor (stride 0) over rows_valid rows of kb bytes starting at
// base: offsets at or past num_records = rows_valid * kb (< 2^31) read as zero.
__device__ __forceinline__ i32x4 tile_rsrc(const int8_t* base, int64_t rows_valid, int64_t kb) {
    const uint64_t b = (uint64_t)base;
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r.z = __builtin_amdgcn_readfirstlane((int)(rows_valid * kb));
    r.w = 0x00020000;
    return r;
}

// An offset past every descriptor's num_records (at most 2^28 bytes where it
// is used): a load from it returns zeros.
constexpr int kOutOfRange = 0x70000000;

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16*lane.
// Written as asm so that the only waits on these loads are the explicit
// s_waitcnt vmcnt(...) placed before the barriers that publish each stage
// (the compiler would otherwise drain every load in flight before reading
// any stage). No register receives the data. The asm sets m0 (the LDS base
// of the load) itself; the compiler warns that it does not preserve m0 across
// the statement, which is harmless here because the generated code of these
// kernels reads m0 nowhere else (no LDS-DMA builtins, GWS, sendmsg or
// interpolation), as the gfx950 assembly of the library shows.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds, int voff, int soff) {
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



// Batched launches: item i owns the blocks [first[i], first[i + 1]) of a
// 1-D grid; the item of block b (uniform per block).
__device__ __forceinline__ int item_of(const int32_t* first, int count, int32_t b) {
    int i = 0;
    while (i + 1 < count && b >= first[i + 1]) ++i;
    return i;
}

}  // namespace sqd
