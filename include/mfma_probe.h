/*
 * mfma_probe.h - matrix-core measurements exported by libattn.so.
 *
 * These calls are the denominators and the evidence behind the attention
 * kernels' figures, not part of the attention path.  The pages state the
 * efficiency of exact attention as a fraction of the chip's theoretical
 * matrix throughput ("FlashAttention-2", Systems analysis wiki, "Performance
 * and efficiency"); attn_mfma_peak measures what the matrix cores of this
 * GPU actually sustain, so a kernel can also be reported against that.
 * attn_mfma_dot exposes how one matrix-core instruction sums its products:
 * the fp8 (e4m3) instruction is used by attn_fwd_fp8 for Q K^T, whose error
 * on inputs with outlier channels ("Scaling FlashAttention, multi-GPU
 * training and weight quantization", itimpress, section 1, FP8 bullet:
 * outliers and incoherent processing) depends on it.
 *
 * Pointers are DEVICE pointers owned by the caller; nothing is allocated;
 * each call enqueues one kernel on `stream` and returns.  Errors are the
 * attn_status codes of attn.h: ATTN_ERR_INVALID for a NULL or misaligned
 * pointer or an out-of-range count, ATTN_ERR_UNSUPPORTED for an unknown
 * kind, ATTN_ERR_HIP for a launch failure.
 */
#ifndef MFMA_PROBE_H
#define MFMA_PROBE_H

#include <stddef.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction kinds. */
#define ATTN_MFMA_BF16 0 /* v_mfma_f32_32x32x16_bf16: 32768 FLOP            */
#define ATTN_MFMA_F16 1  /* v_mfma_f32_32x32x16_f16: 32768 FLOP             */
#define ATTN_MFMA_FP8 2  /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3,
                            unit block scales: 131072 FLOP                  */
#define ATTN_MFMA_F32 3  /* v_mfma_f32_32x32x2_f32: 4096 FLOP (peak only)    */

/* Workgroup size of attn_mfma_peak (8 wavefronts, two per SIMD). */
#define ATTN_MFMA_PEAK_THREADS 512

/* FLOP performed by one attn_mfma_peak launch (0 for invalid arguments). */
double attn_mfma_peak_flop(int kind, int workgroups, int iters);

/*
 * attn_mfma_peak - matrix-core throughput loop.  `workgroups` workgroups of
 * ATTN_MFMA_PEAK_THREADS threads each run `iters` rounds of four independent
 * MFMAs of the given kind on register operands (no memory traffic in the
 * loop).  out: device fp32 [workgroups * ATTN_MFMA_PEAK_THREADS], 4-byte
 * aligned, receives one checksum per thread (its content has no meaning; it
 * keeps the products live).  1 <= workgroups <= 1<<20, 1 <= iters <= 1<<24.
 * The caller times the launch (e.g. with events on `stream`); throughput is
 * attn_mfma_peak_flop(...) / time.
 */
attn_status attn_mfma_peak(int kind, int workgroups, int iters, float* out, void* stream);

/*
 * attn_mfma_dot - C = A B for one 32 x 32 tile with K = 64 on the matrix
 * cores, computed by one wavefront.
 *   kind ATTN_MFMA_FP8: a u8 [32][64] e4m3 codes, row-major; b u8 [32][64]
 *        (column j of B is row j of b); one instruction sums all 64 products
 *        of each output.
 *   kind ATTN_MFMA_BF16 / ATTN_MFMA_F16: a, b 16-bit [32][64] likewise; four
 *        chained 32x32x16 instructions (16 products each) into one fp32
 *        accumulator.
 *   c    fp32 [32][32] row-major, C_ij = sum_k a[i][k] * b[j][k].
 * a and b must be 16-byte aligned, c 4-byte aligned.
 */
attn_status attn_mfma_dot(int kind, const void* a, const void* b, float* c, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MFMA_PROBE_H */
