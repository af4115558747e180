/*
 * sq_ceiling.h -- C ABI of libsq_ceiling: measured ceilings of the MI355X
 * (gfx950) that bound the SmoothQuant W8A8 path's kernels on their rooflines.
 * They are measurement probes, not steps of the method, so they live in a
 * library of their own beside libsq; status codes are libsq's (sq.h).
 *
 * Conventions: device pointers, caller-owned buffers, asynchronous on
 * `stream`, arguments validated before anything is launched (nothing is
 * written on error).
 */
#ifndef SQ_CEILING_H
#define SQ_CEILING_H

#include "sq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * sq_ceiling_mfma runs blocks_per_cu blocks of 4 waves on every compute unit,
 * each wave issuing iters x 8 independent v_mfma_i32_32x32x32_i8 on register
 * operands and nothing else. The operands come from `operands` (device,
 * SQ_CEILING_OPERAND_BYTES, 16-byte aligned, read once per wave): chain c's
 * A operand is bytes (2c)·1024 + lane·16 .. +16, its B operand
 * (2c+1)·1024 + lane·16 .. +16, so the caller chooses the bytes the matrix
 * cores switch (the clock under load depends on them). *ops (host) receives
 * the int8 operations issued (2·32·32·32 per instruction); sink[0] (device,
 * zeroed by the caller) is increased, modulo 2^32, per wave by the sum over
 * chains of element 0 of the accumulator (row 0 of A times column 0 of B: the
 * 32 bytes of lanes 0 and 32 of each operand, paired in order), a check that
 * the loop ran; the caller keeps |that dot product| x iters below 2^31.
 * 1 <= iters <= 2^24, 1 <= blocks_per_cu <= 8 (SQ_ERR_SHAPE otherwise).
 *
 * sq_ceiling_copy copies `bytes` (a multiple of 16; src and dst 16-byte
 * aligned, not overlapping) with 16-byte vector loads and stores only.
 *
 * sq_ceiling_narrow reads src_bytes (a multiple of 16; src 16-byte aligned)
 * and writes src_bytes / 2 to dst (8-byte aligned, not overlapping src): the
 * first 8 bytes of every 16-byte vector, in order. Two bytes read per byte
 * written, the traffic mix of the quantizers.
 *
 * sq_ceiling_read reads `bytes` (a multiple of 16, src 16-byte aligned) with
 * 16-byte vector loads and XORs every 32-bit word read into sink[0] (device,
 * 4-byte aligned; the caller sets its start value), which keeps the loads
 * live and lets the caller check them.
 */
#define SQ_CEILING_OPERAND_BYTES 16384
sq_status sq_ceiling_mfma(int64_t iters, int blocks_per_cu, const void* operands, uint32_t* sink,
                          int64_t* ops, hipStream_t stream);
sq_status sq_ceiling_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);
sq_status sq_ceiling_narrow(const void* src, void* dst, int64_t src_bytes, hipStream_t stream);
sq_status sq_ceiling_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SQ_CEILING_H */
