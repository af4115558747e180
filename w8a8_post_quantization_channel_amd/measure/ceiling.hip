// ceiling.hip -- libsq_ceiling: measured ceilings of MI355X for the roofline
// of the W8A8 path (a library of its own, beside libsq):
// the int8 matrix-core rate of a loop that only issues MFMAs, and the HBM
// rate of a copy that only streams 16-byte vectors. Neither touches the
// method's data; they bound what the GEMM and the HBM passes can reach.
#include <algorithm>

#include "sq_ceiling.h"
#include "sq_device.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kMfmaChains = 8;  // independent accumulators per wave: enough to keep the pipe full

// Every wave issues iters x kMfmaChains v_mfma_i32_32x32x32_i8 on register
// operands loaded once from `operands` (chain c's A operand at byte
// (2c)·1024 + lane·16, its B operand at (2c+1)·1024 + lane·16), so the clock
// under load reflects the bytes the matrix cores switch. Lane 0 of each wave
// adds element 0 of each chain's accumulator (row 0 of A times column 0 of B,
// the bytes of lanes 0 and 32) into sink[0], atomically and modulo 2^32.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, const v4i* __restrict__ operands,
                                                        unsigned* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    v4i a[kMfmaChains], b[kMfmaChains];
    v16i acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) {
        acc[c] = v16i{};
        a[c] = operands[(2 * c) * 64 + lane];
        b[c] = operands[(2 * c + 1) * 64 + lane];
    }
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c], b[c], acc[c], 0, 0, 0);
    }
    unsigned total = 0;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) total += (unsigned)acc[c][0];
    if (lane == 0) atomicAdd(sink, total);
}

constexpr int kCopyUnroll = 8;  // 16-byte vectors per thread per chunk: 32 KiB chunks of 256 threads

// Each block copies whole 32 KiB chunks (grid-stride over chunks), all eight
// loads of a chunk in flight before its stores; non-temporal on both sides.
// The last partial chunk is copied vector by vector.
__global__ __launch_bounds__(256) void copy_kernel(const sqd::u32x4* __restrict__ src, sqd::u32x4* __restrict__ dst,
                                                   int64_t nvec) {
    const int64_t nchunk = nvec / (256 * kCopyUnroll);
    for (int64_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
        const int64_t base = c * (256 * kCopyUnroll) + threadIdx.x;
        sqd::u32x4 t[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) t[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(t[u], dst + base + u * 256);
    }
    for (int64_t i = nchunk * (256 * kCopyUnroll) + (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

// Two bytes read per byte written (the traffic mix of the quantizers): each
// 32 KiB chunk of src gives the first 8 bytes of every 16-byte vector to dst
// (8-byte stores), in the same chunks and with the same loads in flight as
// the copy. The last partial chunk goes vector by vector.
__global__ __launch_bounds__(256) void narrow_kernel(const sqd::u32x4* __restrict__ src, sqd::u32x2* __restrict__ dst,
                                                     int64_t nvec) {
    const int64_t nchunk = nvec / (256 * kCopyUnroll);
    for (int64_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
        const int64_t base = c * (256 * kCopyUnroll) + threadIdx.x;
        sqd::u32x4 t[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) t[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            __builtin_nontemporal_store(sqd::u32x2{t[u][0], t[u][1]}, dst + base + u * 256);
    }
    for (int64_t i = nchunk * (256 * kCopyUnroll) + (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * 256) {
        const sqd::u32x4 t = src[i];
        dst[i] = sqd::u32x2{t[0], t[1]};
    }
}

// Read-only stream over the same chunks: each wave XORs everything it loads
// and lane 0 XORs the wave's word into sink[0], so the loads stay live and
// the caller can check the sum against the XOR of all input words.
__global__ __launch_bounds__(256) void read_kernel(const sqd::u32x4* __restrict__ src, int64_t nvec,
                                                   unsigned* __restrict__ sink) {
    const int64_t nchunk = nvec / (256 * kCopyUnroll);
    unsigned x = 0;
    for (int64_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
        const int64_t base = c * (256 * kCopyUnroll) + threadIdx.x;
        sqd::u32x4 t[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) t[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) x ^= t[u][0] ^ t[u][1] ^ t[u][2] ^ t[u][3];
    }
    for (int64_t i = nchunk * (256 * kCopyUnroll) + (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * 256) {
        const sqd::u32x4 t = src[i];
        x ^= t[0] ^ t[1] ^ t[2] ^ t[3];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x ^= (unsigned)__shfl_xor((int)x, off, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(sink, x);
}

int cus() {
    static int n = [] {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        return c;
    }();
    return n;
}

}  // namespace

namespace {

hipError_t ceiling_mfma(int64_t iters, int blocks_per_cu, const void* operands, unsigned* sink, hipStream_t stream) {
    mfma_loop_kernel<<<dim3((unsigned)(blocks_per_cu * cus())), dim3(256), 0, stream>>>(iters, (const v4i*)operands,
                                                                                        sink);
    return hipGetLastError();
}

int64_t ceiling_mfma_ops(int64_t iters, int blocks_per_cu) {
    return (int64_t)blocks_per_cu * cus() * 4 * kMfmaChains * iters * (2 * 32 * 32 * 32);
}

// Two blocks per compute unit measured fastest for both streams (1 GiB copy:
// 5.6-5.7 TB/s for 2 to 32 blocks per CU within noise; read: 7.1 TB/s).
static unsigned stream_blocks(int64_t nvec) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>((nvec + 255) / 256, (int64_t)cus() * 2));
}

hipError_t ceiling_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t nvec = bytes / 16;
    if (nvec == 0) return hipSuccess;
    copy_kernel<<<dim3(stream_blocks(nvec)), dim3(256), 0, stream>>>((const sqd::u32x4*)src, (sqd::u32x4*)dst, nvec);
    return hipGetLastError();
}

hipError_t ceiling_narrow(const void* src, void* dst, int64_t src_bytes, hipStream_t stream) {
    const int64_t nvec = src_bytes / 16;
    if (nvec == 0) return hipSuccess;
    narrow_kernel<<<dim3(stream_blocks(nvec)), dim3(256), 0, stream>>>((const sqd::u32x4*)src, (sqd::u32x2*)dst,
                                                                       nvec);
    return hipGetLastError();
}

hipError_t ceiling_read(const void* src, int64_t bytes, unsigned* sink, hipStream_t stream) {
    const int64_t nvec = bytes / 16;
    if (nvec == 0) return hipSuccess;
    read_kernel<<<dim3(stream_blocks(nvec)), dim3(256), 0, stream>>>((const sqd::u32x4*)src, nvec, sink);
    return hipGetLastError();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

sq_status hip_status(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

}  // namespace

extern "C" {

sq_status sq_ceiling_mfma(int64_t iters, int blocks_per_cu, const void* operands, uint32_t* sink, int64_t* ops,
                          hipStream_t stream) {
    if (!operands || !sink || !ops) return SQ_ERR_NULL;
    if (iters < 1 || iters > ((int64_t)1 << 24) || blocks_per_cu < 1 || blocks_per_cu > 8) return SQ_ERR_SHAPE;
    if (!aligned16(operands) || ((uintptr_t)sink & 3u) != 0) return SQ_ERR_ALIGN;
    *ops = ceiling_mfma_ops(iters, blocks_per_cu);
    return hip_status(ceiling_mfma(iters, blocks_per_cu, operands, sink, stream));
}

sq_status sq_ceiling_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    if (bytes > 0 && (!src || !dst)) return SQ_ERR_NULL;
    if (bytes < 0 || bytes % 16 != 0) return SQ_ERR_SHAPE;
    if (bytes > 0 && (!aligned16(src) || !aligned16(dst))) return SQ_ERR_ALIGN;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (bytes > 0 && s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return SQ_ERR_SHAPE;
    return hip_status(ceiling_copy(src, dst, bytes, stream));
}

sq_status sq_ceiling_narrow(const void* src, void* dst, int64_t src_bytes, hipStream_t stream) {
    if (src_bytes > 0 && (!src || !dst)) return SQ_ERR_NULL;
    if (src_bytes < 0 || src_bytes % 16 != 0) return SQ_ERR_SHAPE;
    if (src_bytes > 0 && (!aligned16(src) || ((uintptr_t)dst & 7u) != 0)) return SQ_ERR_ALIGN;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst, db = (uintptr_t)(src_bytes / 2);
    if (src_bytes > 0 && s0 < d0 + db && d0 < s0 + (uintptr_t)src_bytes) return SQ_ERR_SHAPE;
    return hip_status(ceiling_narrow(src, dst, src_bytes, stream));
}

sq_status sq_ceiling_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    if (!sink || (bytes > 0 && !src)) return SQ_ERR_NULL;
    if (bytes < 0 || bytes % 16 != 0) return SQ_ERR_SHAPE;
    if ((bytes > 0 && !aligned16(src)) || ((uintptr_t)sink & 3u) != 0) return SQ_ERR_ALIGN;
    return hip_status(ceiling_read(src, bytes, sink, stream));
}

}  // extern "C"
