/*
 * tg_diag.h — measurement aids exported by libtg.so beside the GEMM ABI of
 * tg.h.  Nothing here computes the product; these calls exist so that the
 * GEMM's measured rate can be set against what the matrix cores themselves
 * sustain on the same data.  Same status codes and conventions as tg.h.
 */
#ifndef TG_DIAG_H
#define TG_DIAG_H

#include "tg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---- the matrix cores' rate on given operand values -------------------------
 * No passage of the pages defines this call; it is a measurement aid for the
 * GEMM's roofline.  Under the board's power limit the shader clock drops as
 * the bits of the MFMA operands toggle, so the dense rate that any kernel can
 * sustain depends on the data: all-zero operands reach the nominal peak,
 * random ones stay below it.  This call runs the matrix cores alone on
 * operands taken from `operands`, with no memory traffic in its loop, two
 * waves per SIMD (as in the large GEMM kernels), and so measures the ceiling
 * a GEMM on such values with that MFMA shape can approach.
 *
 * mfma:       32 (v_mfma_f32_32x32x16_f16) or 16 (v_mfma_f32_16x16x32_f16),
 *             the two shapes the fp16 GEMM kernels use, or 64
 *             (v_mfma_i32_16x16x64_i8, the int8 kernels' shape: the operand
 *             bytes are int8 values and a k-step is 64 deep).
 * operands:   TG_CEILING_OPERAND_BYTES bytes of fp16 (int8) values in device
 *             memory (16-byte aligned), read once per thread in 16-byte
 *             chunks: A fragments from the first half of the buffer, B
 *             fragments from the second half (thread t of a workgroup, set
 *             s, block j: A chunk (16 t + 8 s + j) mod 4096, B chunk 4096 +
 *             (8 t + 4 s + j) mod 4096).
 * sink:       workgroups * 512 floats of device memory; thread t of
 *             workgroup w writes the sum of its accumulators to
 *             sink[512 w + t] (so the work is not optimised away).
 * iters:      k-steps of 32 (64) per wave: even, 2 .. 2^30.  The two operand
 *             sets alternate from one k-step to the next.
 * workgroups: 1 .. 2^20 workgroups of 8 waves, two per SIMD; iters *
 *             workgroups at most 2^32 (about ten seconds of work).
 * Work: workgroups * 8 * iters * 2 * 128 * 64 * 32 FLOP (every wave holds a
 * 128 x 64 fp32 accumulator tile); for mfma 64 the last factor is 64 (int8
 * OPs into int32 accumulators).  Asynchronous on `stream`; time it with
 * events on that stream.
 * Errors: TG_ERROR_INVALID_VALUE (bad mfma, iters or workgroups, or too much
 * work; NULL or misaligned pointer; a buffer that does not fit inside its
 * allocation), TG_ERROR_NOT_DEVICE_MEMORY, TG_ERROR_UNSUPPORTED (not gfx950),
 * TG_ERROR_LAUNCH. */
#define TG_CEILING_OPERAND_BYTES 131072
tg_status tg_mfma_ceiling(int mfma, const void *operands, float *sink, int64_t iters,
                          int64_t workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TG_DIAG_H */
