/*
 * sp_ring_attn.h -- C ABI of one rank's ring-attention forward on MI355X
 * (gfx950): context parallelism, the companion of sequence parallelism for
 * the attention core.
 *
 * Context parallelism shards Q, K and V along the sequence: rank i owns a
 * contiguous block of query tokens and the matching K/V block.  Attention
 * needs every key, so the K/V blocks travel around a ring of t ranks; at
 * each step a rank attends its queries to the block in hand and accumulates
 * the partial (online-softmax) result, and after t steps every query has
 * attended every key, with no s x s score matrix ever held ("Sequence
 * parallel math", sections "Where SP stops: the attention core and long
 * sequences" and "Context parallelism and ring attention").  The pages apply
 * no causal mask: every query sees every key.
 *
 * At ring step k (k = 0 .. t-1) rank i holds K/V block (i - k) mod t: its
 * own block first, then each predecessor's.  Per step the library writes
 * the partial result of the block in hand -- O_k = softmax(Q K_k^T * scale)
 * V_k over that block's keys, and its log-sum-exp L_k -- and the merge folds
 * them in ring order, acc = merge(acc, (O_k, L_k)) for k = 0, 1, ..., with
 *   merge((O_a, L_a), (O_b, L_b)) = ((e^{L_a-M} O_a + e^{L_b-M} O_b) / Z,
 *                                    M + log Z),  M = max(L_a, L_b),
 *                                    Z = e^{L_a-M} + e^{L_b-M},
 * which is the whole sequence's attention up to rounding.
 *
 * Conventions:
 *  - Tensors are bf16 (raw 16-bit words), layout [tokens][b][heads][d]
 *    (sequence-major, like the region's [s, b, h] with h = heads*d); lse is
 *    fp32 [s_local][b][heads].  Products run on MFMA with bf16 operands and
 *    fp32 accumulation: the probabilities P are rounded to bf16 before P V,
 *    O is rounded to bf16 once at the end.
 *  - Device pointers 16-byte aligned (lse 4-byte); outputs must not overlap
 *    inputs or each other; the caller owns every buffer, the workspace too.
 *  - Asynchronous on `stream`; errors are found on the host before any
 *    launch, and then nothing is launched.
 */
#ifndef SP_RING_ATTN_H
#define SP_RING_ATTN_H

#include "sp_region.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t s_local;   /* query tokens of this rank = key tokens per block (>= 1) */
    int64_t b;         /* batch (>= 1)                                           */
    int32_t heads;     /* attention heads on this GPU (>= 1; b*heads <= 65535)   */
    int32_t d;         /* head dimension: 64 or 128                              */
    int32_t t;         /* ring size, the context-parallel degree (1 .. 65535)    */
    int32_t rank;      /* this rank, 0 <= rank < t: owns query block `rank`      */
    float   scale;     /* softmax scale; 0 means 1/sqrt(d)                       */
    int32_t steps_per_wg;  /* launch choice for sp_ring_attn_fwd: 0 = the
                              library's own, else k, a divisor of t: each
                              workgroup walks k consecutive ring steps as one
                              run of key tiles and the merge folds t/k
                              partials (same results within the tolerance,
                              deterministic for each k)                      */
} spr_attn_desc;
/* Also rejected (SPR_ERR_INVALID_ARG): ceil(s_local/256) * b * heads * t above
 * 2^31 - 1 (the 256-query tiles of all steps form one launch). */

/* Bytes of workspace for the t partial results: fp32 O_k [t][s_local][b]
 * [heads][d] and L_k [t][s_local][b][heads].  0 on an invalid desc. */
size_t sp_ring_attn_workspace_bytes(const spr_attn_desc* desc);

/* The whole forward of rank `rank` with every K/V block resident (one GPU
 * simulating the ring): all t steps, then the merge.
 *  q     [s_local][b][heads][d]        this rank's queries
 *  k, v  [t][s_local][b][heads][d]     block j = the tokens of rank j
 *  o_out [s_local][b][heads][d] bf16   attention output
 *  lse_out [s_local][b][heads] fp32    log-sum-exp of the scaled scores, may be NULL */
spr_status sp_ring_attn_fwd(const spr_attn_desc* desc, const void* q, const void* k,
                            const void* v, void* o_out, float* lse_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* One ring step: the partial result of the block in hand, k_blk and v_blk
 * ([s_local][b][heads][d], block (rank - step) mod t), into slot `step` of
 * the workspace.  Steps may run in any order or concurrently (they write
 * different slots); sp_ring_attn_merge then folds slots 0 .. t-1. */
spr_status sp_ring_attn_step(const spr_attn_desc* desc, int32_t step, const void* q,
                             const void* k_blk, const void* v_blk, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
spr_status sp_ring_attn_merge(const spr_attn_desc* desc, void* o_out, float* lse_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* sp_ring_attn_fwd is two kernel launches on `stream`: the ring steps (index
 * 0; each workgroup may walk several consecutive steps and write one partial
 * for them), then the merge of those partials (index 1).  These two let a
 * caller run them one at a time -- to time each kernel with events on the
 * stream; launching indices 0 and 1 in order on one stream is exactly
 * sp_ring_attn_fwd.  Same arguments and checks as sp_ring_attn_fwd.
 * sp_ring_attn_fwd_num_launches returns 0 for an invalid desc;
 * sp_ring_attn_fwd_launch returns SPR_ERR_INVALID_ARG for an index outside
 * 0 .. n-1 (after the other checks, before any launch). */
int sp_ring_attn_fwd_num_launches(const spr_attn_desc* desc);
spr_status sp_ring_attn_fwd_launch(const spr_attn_desc* desc, int index, const void* q,
                                   const void* k, const void* v, void* o_out, float* lse_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SP_RING_ATTN_H */
