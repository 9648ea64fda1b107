/*
 * attn.h - C ABI of libattn.so: exact, IO-aware softmax attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes O = softmax(scale * Q K^T [+ causal mask]) V together
 * with the per-row log-sum-exp, tile by tile with an online softmax, so the
 * Nq x Nk score matrix never reaches device memory.  The operation is standard
 * softmax attention, reached exactly up to floating-point rounding
 * ("FlashAttention-2", Systems analysis wiki: lead paragraph, "Background: the
 * attention problem in transformers", "Technical architecture and working
 * principles"); the block-wise state merge is the online softmax of
 * "Sequence parallelism and ring attention" (aiunderstanding.org, "Deep dive",
 * "Technical insight"); the fp8 entry point takes the block-quantized inputs
 * of "Scaling FlashAttention, multi-GPU training and weight quantization"
 * (itimpress, section 1, FP8 bullet).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller (except the
 *    host-resident K/V blocks of attn_fwd_ring_host).  The library allocates no
 *    memory and never synchronises the host: each call validates its arguments
 *    on the host, enqueues its kernels on `stream` (a hipStream_t; NULL means
 *    the default stream) and returns.  Global state is limited to three caches
 *    that live until the process ends and never change a result: each device's
 *    compute-unit count (read once, used to size the W4A16 grid and the bf16
 *    forward's persistent grid), attn_fwd_ring_host's per-device copy stream
 *    with five events, and attn_bwd's per-device side stream with two events;
 *    each stream is created on its entry point's first call on the device and
 *    guarded by a mutex, and work on it is joined back to `stream` before the
 *    call returns.
 *  - Layout: contiguous [B, H, N, d] row-major, d innermost; per-row outputs
 *    (lse, m, l) are contiguous [B, H, N].  Q/K/V/O pointers must be 16-byte
 *    aligned; per-row pointers 4-byte aligned.  Outputs must not alias inputs.
 *  - d must be 64 or 128.  B, H, N >= 1.  `scale` must be finite (any sign;
 *    0 gives uniform weights).
 *  - Scores are s_ij = scale * q_i . k_j.  With `causal` set, query row i may
 *    attend key j iff j <= i + (Nk - Nq) (bottom-right aligned; j <= i when
 *    Nq == Nk).  A row with no allowed key gets O = 0 and lse = -inf.
 *  - lse_i = ln sum_j exp(s_ij) over the allowed keys (natural log, includes
 *    scale), in fp32.
 *  - Errors: arguments are checked before anything is enqueued.  A failed
 *    check returns ATTN_ERR_INVALID (null pointer, non-positive size,
 *    misalignment, non-finite scale, size overflow) or ATTN_ERR_UNSUPPORTED
 *    (a d other than 64/128) and launches nothing, writes nothing.  If the HIP
 *    runtime reports an error at launch, ATTN_ERR_HIP is returned; outputs are
 *    then undefined.  Kernel faults surface at the caller's next
 *    synchronisation, as for any HIP kernel.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    (no atomics, fixed reduction order).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1
/* Tokens per quantization tile of attn_fwd_fp8 scales. */
#define ATTN_FP8_TILE 128

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,
    ATTN_ERR_UNSUPPORTED = 2,
    ATTN_ERR_HIP = 3
} attn_status;

/* Constant ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

/* Static, human-readable name of a status code. */
const char* attn_status_str(attn_status s);

/*
 * attn_fwd - one pass over all keys, bfloat16 in, bfloat16 out.
 *   q   bf16 [B,H,Nq,d]     k, v  bf16 [B,H,Nk,d]
 *   o   bf16 [B,H,Nq,d]     O = P V with P = softmax of the allowed scores,
 *                           accumulated in fp32, rounded to nearest-even once.
 *   lse fp32 [B,H,Nq]       may be NULL (not written).
 * The outer loop runs over 256-row query blocks, spread over all compute
 * units (sequence-length parallelism): one persistent workgroup of 8
 * wavefronts per compute unit walks its share of the blocks, longest first;
 * the inner loop streams 128-key K/V tiles through LDS (double buffered, the
 * stream running on across block boundaries), keeps the running max /
 * normaliser per row and divides by the normaliser once after the loop
 * ("FlashAttention-2", Systems analysis wiki, "Technical architecture and
 * working principles", items 1-3).  Causal key tiles above the diagonal are
 * skipped wholesale.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Nq, int Nk, int d, int causal, float scale,
                     void* stream);

/*
 * attn_fwd_f32 - as attn_fwd with float32 q/k/v/o (fp32 matrix-core products,
 * fp32 probabilities).  lse may be NULL.
 */
attn_status attn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                         float* lse, int B, int H, int Nq, int Nk, int d, int causal,
                         float scale, void* stream);

/*
 * attn_fwd_kvblock - partial attention of the local queries against one block
 * of keys/values: the per-hop compute of ring attention on one GPU
 * ("Sequence parallelism and ring attention", "Deep dive", "Technical insight").
 *   q       bf16 [B,H,Nq,d]           k_blk, v_blk  bf16 [B,H,Nk_blk,d]
 *   o_part  fp32 [B,H,Nq,d]  O of the block, normalised by its own l
 *   m_part  fp32 [B,H,Nq]    max_j s_ij over the block's allowed keys
 *                            (natural units, includes scale); -inf if none
 *   l_part  fp32 [B,H,Nq]    sum_j exp(s_ij - m_part); 0 if no key allowed
 * q_pos0 / k_pos0 are the global token positions of query row 0 and of the
 * block's key 0; with `causal` set key j is allowed for row i iff
 * k_pos0 + j <= q_pos0 + i (ignored when causal == 0).  A row with no allowed
 * key gets the empty state (O = 0, m = -inf, l = 0), the identity of
 * attn_merge.
 */
attn_status attn_fwd_kvblock(const void* q, const void* k_blk, const void* v_blk,
                             float* o_part, float* m_part, float* l_part,
                             int B, int H, int Nq, int Nk_blk, int d, int causal,
                             int64_t q_pos0, int64_t k_pos0, float scale, void* stream);

/*
 * attn_merge - online-softmax merge of a block state into an accumulated
 * state, in place:  M = max(m_acc, m_part); w_x = l_x exp(m_x - M);
 * o_acc = (w_acc o_acc + w_part o_part) / (w_acc + w_part); l_acc = w_acc +
 * w_part; m_acc = M.  The empty state (m = -inf, l = 0) is the identity.
 *   o_acc, o_part  fp32 [B,H,Nq,d]     m_*, l_*  fp32 [B,H,Nq]
 *   o_final        bf16 [B,H,Nq,d] or NULL: if given, also receives the
 *                  merged O rounded to bf16
 *   lse_final      fp32 [B,H,Nq] or NULL: if given, receives M + ln l
 *                  (-inf for the empty state)
 * The accumulator is always updated.  To start an accumulation, either
 * write the first block's attn_fwd_kvblock output straight into the
 * accumulator, or initialise m = -inf, l = 0, o = 0.
 * o_acc/m_acc/l_acc may not alias the *_part buffers.  Here d may be any
 * multiple of 4 in [4, 1024].
 */
attn_status attn_merge(float* o_acc, float* m_acc, float* l_acc,
                       const float* o_part, const float* m_part, const float* l_part,
                       void* o_final, float* lse_final,
                       int B, int H, int Nq, int d, void* stream);

/*
 * attn_bwd - gradients of L = sum(dO * O) with respect to q, k and v for the
 * attention that attn_fwd computes, from its output and log-sum-exp; the
 * probabilities are recomputed tile by tile and never stored.  The pages give
 * training results that presuppose this pass ("FlashAttention-2",
 * "Performance and efficiency"; the FlashAttention-4 summary's training
 * backward) but no formula: it is the chain rule applied to the forward,
 *   P = exp(scale q.k - LSE),  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),
 *   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *   q, o, dout      bf16 [B,H,Nq,d]     k, v  bf16 [B,H,Nk,d]
 *   lse             fp32 [B,H,Nq]  as attn_fwd writes it (natural log,
 *                   including scale; -inf for rows without keys)
 *   dq              bf16 [B,H,Nq,d]     dk, dv  bf16 [B,H,Nk,d]  (outputs)
 *   work            device fp32 workspace of attn_bwd_work_floats(B,H,Nq)
 *                   floats (receives D), owned by the caller
 * causal and scale as in attn_fwd (any finite scale).  Products run on bf16
 * matrix cores with fp32 accumulation; P and dS are rounded to bf16 for them.
 * The dQ kernel runs on the library's side stream for the device, after D is
 * written and concurrently with the dK/dV kernel; `stream` waits for it, so
 * every output is complete for work enqueued on `stream` after the call.
 * Errors: as attn_fwd, plus ATTN_ERR_INVALID for a NULL lse or work.
 */
size_t attn_bwd_work_floats(int B, int H, int Nq);
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     float* work, int B, int H, int Nq, int Nk, int d, int causal,
                     float scale, void* stream);

/*
 * attn_fwd_ring - one GPU's whole share of ring attention ("Sequence
 * parallelism and ring attention", "Deep dive" and "Technical insight"):
 * the local query shard against the K/V blocks that the ring's hops deliver,
 * in hop order, each block's partial state (as attn_fwd_kvblock) folded into
 * a running state (as attn_merge; after the first block the fold happens in
 * the attention kernel's epilogue, so block states never round-trip through
 * memory), then the final bf16 O and LSE.
 *   q       bf16 [B,H,Nq,d], query row i at global position q_pos0 + i
 *   k_blks, v_blks   HOST arrays of n_blk device pointers, each block
 *                    bf16 [B,H,Nk_blk,d]; block b's key j sits at global
 *                    position k_pos[b] + j (k_pos: HOST array of n_blk)
 *   o       bf16 [B,H,Nq,d]      lse  fp32 [B,H,Nq] natural log, or NULL
 *   work    device fp32 workspace of attn_ring_work_floats(B,H,Nq,d)
 *           floats (B*H*Nq*(d+2): the running O, m and l), 16-byte aligned,
 *           owned by the caller; its contents on return are unspecified.  It
 *           must not overlap any other argument.
 * With `causal` set, key position kp is allowed for query position qp iff
 * kp <= qp; a block whose first key lies after the shard's last row holds no
 * allowed key and is skipped without a launch.  n_blk = 0, or every block
 * skipped, gives O = 0 and LSE = -inf.  The blocks must already be resident
 * on this device: the library moves no data between GPUs.
 * Errors: as attn_fwd_kvblock, plus ATTN_ERR_INVALID for n_blk < 0, NULL
 * arrays with n_blk > 0, a NULL or misaligned block, or a negative position
 * with `causal` set.  Arguments are all checked before the first launch; a
 * launch failure returns ATTN_ERR_HIP with the earlier steps enqueued.
 */
size_t attn_ring_work_floats(int B, int H, int Nq, int d);
attn_status attn_fwd_ring(const void* q, const void* const* k_blks, const void* const* v_blks,
                          const int64_t* k_pos, int n_blk, void* o, float* lse, float* work,
                          int B, int H, int Nq, int Nk_blk, int d, int causal, int64_t q_pos0,
                          float scale, void* stream);

/*
 * attn_fwd_ring_host - attn_fwd_ring with the K/V blocks arriving from HOST
 * memory, the block transfer overlapped with the attention of the previous
 * block ("Sequence parallelism and ring attention", "Deep dive": the K/V
 * exchange of the ring runs under the computation, so it adds little wall
 * time).  On one GPU the host link stands in for the ring's peer link.
 *   k_blks, v_blks   HOST arrays of n_blk HOST pointers, each block bf16
 *                    [B,H,Nk_blk,d] in host memory.  Page-locked memory
 *                    (hipHostMalloc) is needed for the copies to run
 *                    asynchronously; pageable memory gives the same result
 *                    with the copies serialised against the host thread.
 *   stage   device buffer of attn_ring_stage_bytes(B,H,Nk_blk,d) bytes,
 *           16-byte aligned, owned by the caller: two slots, each one
 *           block's K then V.  Contents on return are unspecified.
 *   other arguments as attn_fwd_ring.
 * Live block i (blocks skipped by the causal rule are neither copied nor
 * computed) is copied into slot i % 2 on a copy stream that the library
 * keeps per device; its attention runs on `stream` once the copy is done,
 * and the copy of live block i + 2 waits until that attention has finished
 * reading the slot.  The first copy also waits for the work enqueued on
 * `stream` before the call.  All of the call's work, copies included, is
 * complete once `stream` reaches the point of the call's return; the host
 * blocks must stay valid and unchanged until then.  The result is
 * bit-identical to attn_fwd_ring on the same blocks resident on the device.
 * Calls from several host threads are serialised inside the library.
 * Errors: as attn_fwd_ring (a NULL block pointer is ATTN_ERR_INVALID), plus
 * ATTN_ERR_INVALID for a NULL or misaligned `stage`, or one that overlaps
 * `work`; ATTN_ERR_HIP if the copy stream or a copy fails.
 */
size_t attn_ring_stage_bytes(int B, int H, int Nk_blk, int d);
attn_status attn_fwd_ring_host(const void* q, const void* const* k_blks, const void* const* v_blks,
                               const int64_t* k_pos, int n_blk, void* o, float* lse, float* work,
                               void* stage, int B, int H, int Nq, int Nk_blk, int d, int causal,
                               int64_t q_pos0, float scale, void* stream);

/*
 * attn_fwd_fp8 - attention on block-quantized OCP FP8 E4M3 ("e4m3fn") inputs
 * ("Scaling FlashAttention, multi-GPU training and weight quantization",
 * itimpress, section 1, FP8 bullet: a separate scale per small tile).
 *   q8   u8 [B,H,Nq,d]   k8, v8  u8 [B,H,Nk,d]      e4m3 codes
 *   q_scale fp32 [B,H,ceil(Nq/128)]   k_scale, v_scale fp32 [B,H,ceil(Nk/128)]
 *        the value of element x of token n is code(x) * scale[b,h,n/128]
 *   o    fp32 [B,H,Nq,d]     lse fp32 [B,H,Nq] or NULL
 * Q K^T runs on fp8 matrix cores; P V runs with P in fp16 against V codes
 * converted exactly to fp16; O is kept and written in fp32.
 * The fp8 matrix cores sum the products of one instruction with limited
 * alignment precision, so a channel whose products dwarf the others (an
 * outlier channel) perturbs the scores; the same passage's remedy,
 * "incoherent processing" (Q and K multiplied by one random orthogonal
 * matrix before quantization), removes such channels.  attn_fwd_fp8_qk16
 * below is exact for any codes.
 * Scales must be finite and > 0; NaN codes (0x7F, 0xFF) give undefined output.
 */
attn_status attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         float* o, float* lse, int B, int H, int Nq, int Nk, int d,
                         int causal, float scale, void* stream);

/*
 * attn_fwd_fp8_qk16 - attn_fwd_fp8 with Q K^T on fp16 matrix cores over the
 * codes widened exactly to fp16 (exact products, fp32 sums), for
 * block-quantized inputs that were not rotated.  Same arguments, layout and
 * outputs as attn_fwd_fp8; the fp8 storage (half the bytes of bf16) is kept.
 */
attn_status attn_fwd_fp8_qk16(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                              const float* q_scale, const float* k_scale, const float* v_scale,
                              float* o, float* lse, int B, int H, int Nq, int Nk, int d,
                              int causal, float scale, void* stream);

/*
 * attn_fwd_fp8_pv8 - as attn_fwd_fp8 with the probabilities in e4m3 too:
 * both products on the fp8 matrix cores (the FlashAttention-3 FP8 form,
 * "Scaling FlashAttention, multi-GPU training and weight quantization" §1),
 * V's codes used as they are.  P is quantized as p * s_v / max s_v * 2^8 and
 * the matrix core's block scale 2^-8 undoes the factor exactly; the
 * normaliser sums the rounded values.  e4m3 keeps 3 mantissa bits, so the
 * result drifts from exact attention by the rounding of P: a speed-for-
 * accuracy mode (the drift is measured and reported, not held to the fp8
 * parity bar).  Same arguments and errors as attn_fwd_fp8; for inputs with
 * outlier channels apply the rotation, as for attn_fwd_fp8.
 */
attn_status attn_fwd_fp8_pv8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             float* o, float* lse, int B, int H, int Nq, int Nk, int d,
                             int causal, float scale, void* stream);

/*
 * attn_fwd_fp8_pv4 - as attn_fwd_fp8_pv8 with the probabilities as 4-bit
 * e2m1 codes ("Hardware-Aware FP4 FlashAttention-4", gist.science summary:
 * probabilities kept in the hardware's 4-bit format for the P.V product).
 * P is quantized as 4 p s_v / max s_v (at most 4) and the matrix core's
 * block scale 2^-2 undoes the factor; P.V runs on the f8f6f4 matrix cores
 * with V's e4m3 codes; the normaliser sums the decoded codes.
 *   direct_p = 0: each exponential is rounded to e2m1 (nearest even).
 *   direct_p = 1: Direct-P: the score's base-2 exponent relative to the
 *     running maximum is mapped straight to the code index (no
 *     exponential): index = clamp(round(2 log2(4 p') + 2), 0, 6), which
 *     matches nearest-even rounding for 4 p' >= 0.59 and flushes smaller
 *     values to 0.
 * e2m1 has one mantissa bit and nothing below 0.5 but 0: probabilities
 * below 1/16 (1/8 rounded) of the row maximum vanish and the others move by
 * up to 1/3; a speed-for-accuracy mode whose drift is measured, not held to
 * the parity bar.  Same arguments and errors as attn_fwd_fp8, plus
 * ATTN_ERR_INVALID for direct_p other than 0 or 1.
 */
attn_status attn_fwd_fp8_pv4(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             float* o, float* lse, int B, int H, int Nq, int Nk, int d,
                             int causal, float scale, int direct_p, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
