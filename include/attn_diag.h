/*
 * attn_diag.h - diagnostic entry point of libattn.so: attn_fwd with a
 * different assignment of work to workgroups.
 *
 * The pages describe exact attention as deterministic ("FlashAttention-2",
 * Systems analysis wiki, "Performance and efficiency"): the result may not
 * depend on the order in which the hardware runs the workgroups.  In
 * attn_fwd every output row is computed by one workgroup with a fixed
 * reduction order, and no workgroup reads another's results; this entry
 * point lets a test reorder the work and check that the output stays
 * bit-identical.  It is not meant for production use (the order it sets
 * gives up the placement of each (b, h) slice on one XCD's L2).
 *
 * Conventions of attn.h apply (device pointers owned by the caller, no
 * allocation, no host synchronisation, arguments checked before anything
 * is enqueued).
 */
#ifndef ATTN_DIAG_H
#define ATTN_DIAG_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_fwd_block_order - attn_fwd (same arguments, errors and result) with
 * the workgroup that computes each (b, h, query block) tile chosen by a
 * bijection seeded by `order`: workgroup g takes tile (g * mul + add) mod G,
 * G the grid size, mul coprime to G, both derived from `order` on the host.
 * order = 0 is attn_fwd's own assignment.
 */
attn_status attn_fwd_block_order(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int H, int Nq, int Nk, int d, int causal, float scale,
                                 uint32_t order, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DIAG_H */
