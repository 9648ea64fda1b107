/*
 * w4a16.h - C ABI of libattn.so's W4A16 linear layer: 16-bit activations
 * times 4-bit weights dequantized on the fly, on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one of "Scaling FlashAttention, multi-GPU training and
 * weight quantization" (itimpress), section 3, on-the-fly dequantization
 * (W4A16): weights stored as 4-bit integers, eight to a 32-bit word, read
 * from HBM in that form, widened in registers with shifts and masks using a
 * stored scale and zero point, and multiplied with fp16 activations on the
 * matrix cores; the widened weights are never written to memory.
 *
 *   y[m][n] = sum_k x[m][k] * (q[n][k] - zeros[n][k/group]) * scales[n][k/group]
 *
 * Format (the page does not fix the order of the eight codes in a word; this
 * is the library's choice):
 *   x       fp16 [M, K] row-major                       16-byte aligned
 *   packed  u32  [N, K/8]; code q[n][8j + e] is bits 4*(e/2) + 16*(e%2) .. +3
 *           of packed[n][j] (even e in the low half-word, odd e in the high
 *           one, in order)                              16-byte aligned
 *   scales  fp16 [N, K/group]                           2-byte aligned
 *   zeros   u8   [N, K/group], each 0..15 (larger values are taken as given)
 *   y       fp16 [M, N] row-major, written              2-byte aligned
 * Conventions of attn.h apply: device pointers owned by the caller, nothing
 * allocated, no host synchronisation, work enqueued on `stream` (a
 * hipStream_t, NULL = default stream), deterministic results, arguments
 * checked before anything is enqueued, outputs must not alias inputs.
 *
 * Arithmetic: the fp16 products run on the matrix cores with fp32
 * accumulation; every widened weight is exact in fp16 and the scale is
 * applied once per group to the fp32 partial sum; y is rounded to fp16
 * (nearest even) once at the end.
 */
#ifndef W4A16_H
#define W4A16_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Codes per group (the only group size the kernels take). */
#define W4A16_GROUP 128
/* Tokens per pass over W (one MFMA block of tokens).  A call with M > 16
 * makes ceil(M / 16) passes, reading W once per pass: the kernels are built
 * for decoding (M <= 16), where W is read exactly once. */
#define W4A16_TOKENS_PER_PASS 16
/* Largest token count M of one call. */
#define W4A16_MAX_M 4096

/*
 * w4a16_work_floats - fp32 workspace that w4a16_gemm needs for these sizes
 * (0 when none; long K is cut into splits whose partial sums meet there).
 * Depends on the sizes only, not on the device.  Returns 0 for sizes that
 * w4a16_gemm would reject.
 */
size_t w4a16_work_floats(int64_t M, int64_t N, int64_t K, int64_t group);

/*
 * w4a16_gemm - y = x . W^T for the 4-bit weight matrix W described above.
 *   work    device fp32 workspace of w4a16_work_floats(M, N, K, group)
 *           floats, 4-byte aligned, owned by the caller (may be NULL when
 *           that is 0); its contents on return are unspecified.  It must not
 *           overlap any other argument.
 * Errors: ATTN_ERR_INVALID for a NULL or misaligned pointer, M, N or K < 1,
 * K not a multiple of group, N > 2^30, K > 2^24, or a NULL or misaligned work
 * when one is needed; ATTN_ERR_UNSUPPORTED for group != W4A16_GROUP or
 * M > W4A16_MAX_M.  Nothing is enqueued when a check fails.  ATTN_ERR_HIP if
 * the runtime reports a launch error.
 */
attn_status w4a16_gemm(const void* x, const uint32_t* packed, const void* scales,
                       const uint8_t* zeros, void* y, float* work, int64_t M, int64_t N,
                       int64_t K, int64_t group, void* stream);

/* Largest split workspace (fp32 elements, 8 MiB) that w4a16_gemm_noalloc
 * holds in its fixed device array. */
#define W4A16_NOALLOC_MAX_WORK_FLOATS (1u << 21)

/*
 * w4a16_gemm_noalloc - w4a16_gemm for callers that cannot allocate device
 * memory or pass a workspace (code under stream capture, tight decode loops,
 * harnesses that forbid allocation).  Same arguments, layout, result (bit
 * for bit) and errors as w4a16_gemm, without `work`: the split partials go to
 * a fixed device array of W4A16_NOALLOC_MAX_WORK_FLOATS floats that the
 * library keeps on each GPU it runs on until the process ends.  Calls whose
 * w4a16_work_floats exceeds that limit return ATTN_ERR_UNSUPPORTED and
 * enqueue nothing; calls that need no split do not touch the array.  The
 * call allocates nothing (its first call on a device looks up the array's
 * device address once).  Every call on one GPU shares the one array, so
 * calls that may overlap on the same GPU (different streams, or host threads
 * without ordering) race and give undefined results; calls ordered on one
 * stream are safe.  ATTN_ERR_HIP if the array's address cannot be obtained.
 */
attn_status w4a16_gemm_noalloc(const void* x, const uint32_t* packed, const void* scales,
                               const uint8_t* zeros, void* y, int64_t M, int64_t N, int64_t K,
                               int64_t group, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
