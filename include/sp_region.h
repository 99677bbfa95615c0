/*
 * sp_region.h -- C ABI of the MI355X (gfx950) sequence-parallel region library.
 *
 * One rank's token shard [s/t, b, h] of a transformer layer's block-boundary
 * activation goes through the band that Megatron-style sequence parallelism
 * shards along the sequence: the reduced row-parallel output x gets a bias,
 * residual dropout, the residual add, and the next LayerNorm (or RMSNorm).
 *
 *   forward   u = x + bias ; keep = Philox(e) >= floor(p * 2^32)
 *             h = residual + (keep ? u * 1/(1-p) : 0)      (rounded to the I/O type)
 *             y = Norm(h) * gamma (+ beta)
 *   backward  dh = Norm'(h)^T (dy * gamma) + dh_out ; dresidual = dh
 *             dx = keep ? dh / (1-p) : 0 ; dgamma, dbeta, dbias = column sums
 *
 * Sources, by page title and section:
 *  - "Sequence parallel math": rank i owns tokens [i*s/t, (i+1)*s/t) ("The
 *    one-line idea"); LayerNorm is per token and residual dropout elementwise,
 *    so a shard computes exactly its slice of the unsharded result ("The move:
 *    split the LayerNorm/dropout band along the sequence"); the band keeps
 *    the two LayerNorm inputs, the two dropout masks and the block inputs,
 *    10*s*b*h replicated under TP and 10*s*b*h/t under SP ("What tensor
 *    parallelism leaves replicated", "The activation-memory saving, in one
 *    formula").
 *  - "Tensor and sequence parallelism -- explained with pictures": a
 *    sub-block has LayerNorm at its entrance, dropout on its output and a
 *    residual from its input ("Transformer block"); after the reduce-scatter
 *    each device applies dropout locally ("Add Sequence parallelism").
 *  - "SP: Partition Activations Alongside TP": RMSNorm rescales a token from
 *    its own features and the residual shares the token layout ("Normalize
 *    and add residuals by token"); after reduce-scatter the SP region adds
 *    the residual and normalises again ("Connect SP and TP across a layer").
 *
 * Readings where the pages are silent: bias is an fp32 [h] vector added
 * before dropout (NULL = zero); dropout is inverted, scale = fp32(1/(1-p));
 * the generator is Philox4x32-10 (Salmon et al., SC'11) with key (seed lo,
 * seed hi) and counter (e/4 lo, e/4 hi, offset lo, offset hi), element e
 * taking word e mod 4, where e = (shard_index*N + r)*h + c is the element's
 * index in the FULL [s, b, h] tensor -- a shard draws exactly what the
 * unsharded run draws; keep iff word >= floor(p*2^32); p == 0 keeps all and
 * writes no mask; the mask is one byte per element, 1 = keep; h is rounded
 * to the I/O type (round to nearest even) before the norm reads it;
 * LayerNorm uses the population variance with eps inside the square root;
 * RMSNorm is y = gamma*h/sqrt(mean(h^2)+eps) with no beta.
 *
 * Conventions for every entry point:
 *  - N = s_local*b token rows; every per-token tensor is contiguous
 *    row-major [N, h] (the shard of a sequence-major [s, b, h] tensor).
 *  - I/O tensors (x, residual, h, y, dy, dh_out, dx, dresidual) have the
 *    element type desc->io: IEEE binary32, or bfloat16 as raw 16-bit words.
 *    bias, gamma, beta, mean, rstd, dgamma, dbeta, dbias are always fp32.
 *  - All pointers are DEVICE pointers (any hipMalloc'd / torch CUDA memory
 *    of the current device), except desc and the byte-count outputs, which
 *    are host pointers.  I/O tensors and bias/gamma/beta must be 16-byte
 *    aligned, mask 8-byte aligned, statistics and gradients 4-byte aligned.
 *  - h must be a multiple of 8 (bf16) or 4 (fp32), and a row at most 4096
 *    such 16-byte vectors: h <= 32768 (bf16), h <= 16384 (fp32).
 *  - Outputs must not overlap inputs or each other.
 *  - The caller owns every buffer, the workspace included; the library never
 *    allocates or frees memory and keeps no state between calls.
 *  - Calls are asynchronous on `stream` (NULL = the null stream): they
 *    return after the launches and the outputs are valid once the stream
 *    has reached that point.
 *  - Errors: every argument is checked on the host before anything is
 *    launched (only device queries -- the compute-unit count, a kernel's
 *    occupancy -- may run first); on an error nothing is launched and no
 *    output is touched.  SPR_ERR_HIP means a HIP call failed (the HIP error
 *    is consumed); outputs are then undefined.
 */
#ifndef SP_REGION_H
#define SP_REGION_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPR_OK = 0,
    SPR_ERR_INVALID_ARG = 1,   /* a NULL/misaligned/overlapping pointer or a bad field */
    SPR_ERR_UNSUPPORTED = 2,   /* valid but not handled: h not a multiple of the vector, h too wide */
    SPR_ERR_WORKSPACE = 3,     /* workspace missing or smaller than sp_region_bwd_workspace_bytes */
    SPR_ERR_HIP = 4            /* a HIP launch or query failed */
} spr_status;

typedef enum { SPR_F32 = 0, SPR_BF16 = 1 } spr_dtype;
typedef enum { SPR_LAYERNORM = 0, SPR_RMSNORM = 1 } spr_norm;

/* Shard shape and region settings. */
typedef struct {
    int64_t  s_local;      /* tokens of this shard along the sequence, s/t (>= 1)   */
    int64_t  b;            /* batch (>= 1)                                          */
    int64_t  h;            /* hidden size                                           */
    int32_t  shard_index;  /* this rank's position in the sequence, 0 <= i < t      */
    int32_t  t;            /* sequence/tensor-parallel degree (>= 1)                */
    int32_t  io;           /* spr_dtype of the I/O tensors                          */
    int32_t  norm;         /* spr_norm                                              */
    float    p;            /* dropout probability, 0 <= p < 1                       */
    float    eps;          /* > 0, finite                                           */
    uint64_t seed;         /* dropout key                                           */
    uint64_t offset;       /* dropout stream, one per dropout site (e.g. 2*layer+k) */
    /* Launch choices; 0 everywhere = the library's own (the usual setting).
     * They select which kernels run, never what is computed: masks and h are
     * the same bits under every choice, the rest meets the same tolerances,
     * and every choice is deterministic.  Out-of-range values are
     * SPR_ERR_INVALID_ARG. */
    int32_t  fwd_kernel;     /* SPR_FWD_AUTO, SPR_FWD_ROWS (one team per row), or
                                SPR_FWD_STREAM (a chip-filling grid walking rows;
                                where it has no plan -- rows of <= 2048 bf16 / 1024
                                fp32 elements or > 16 elements per thread -- and in
                                sp_region_fwd_rs the row kernel runs)            */
    int32_t  bwd_path;       /* SPR_BWD_AUTO, SPR_BWD_FUSED (one row pass, where a
                                row team's column sums fit in registers; else the
                                split passes run), or SPR_BWD_SPLIT (a row-sum pass,
                                then column tiles)                               */
    int32_t  bwd_tile_rows;  /* 0, or rows per tile of the split backward's second
                                pass and of sp_region_bwd_exit: a multiple of 16 in
                                [16, 2^20] (raised to fit 65535 row blocks)      */
    int32_t  reserved;       /* must be 0                                        */
} spr_desc;

enum { SPR_FWD_AUTO = 0, SPR_FWD_ROWS = 1, SPR_FWD_STREAM = 2 };
enum { SPR_BWD_AUTO = 0, SPR_BWD_FUSED = 1, SPR_BWD_SPLIT = 2 };

/* Forward of the region on one shard.
 *  x        [N,h] io   the reduce-scattered row-parallel output
 *  bias     [h]  fp32  may be NULL (same as zero)
 *  residual [N,h] io   the residual stream entering the region
 *  gamma    [h]  fp32
 *  beta     [h]  fp32  LayerNorm: required; RMSNorm: must be NULL
 *  h_out    [N,h] io   residual + dropout(x + bias): the next residual and
 *                      the norm input kept for the backward
 *  y_out    [N,h] io   Norm(h): the input of the next tensor-parallel block
 *  mask_out [N,h] u8   1 = kept; ignored (may be NULL) when p == 0.  With
 *                      p > 0 it may also be NULL: then no mask is stored
 *                      and the backward regenerates the decisions from the
 *                      same generator words (pass mask = NULL there too);
 *                      this keeps N*h bytes fewer per call for extra
 *                      arithmetic in the backward (a mask-free region, the
 *                      trade-off the pages' accounting of the masks invites:
 *                      "Sequence parallel math", "What tensor parallelism
 *                      leaves replicated")
 *  mean_out [N]  fp32  LayerNorm: required; RMSNorm: must be NULL
 *  rstd_out [N]  fp32  1/sqrt(var + eps) (LayerNorm) or 1/sqrt(mean(h^2)+eps)
 * h_out and mask_out are bit-exact functions of the inputs; y and the
 * statistics are computed in fp32.
 *
 * The two ends of the layer stack ("Tensor and sequence parallelism --
 * explained with pictures", section "Transformer block": a sub-block has a
 * LayerNorm at its entrance and a dropout and residual add at its exit):
 *  - x == NULL, the norm-only entry (the first block's norm, with no
 *    branch before it): h is the residual bit for bit and y = Norm(residual).
 *    p must be 0 and bias NULL; h_out may be NULL (h is then not written:
 *    the caller's residual is h, and the backward reads it as h).
 *  - gamma == NULL, the norm-free exit (the last residual add, with no norm
 *    after it): only h and the mask are written; beta, y_out, mean_out and
 *    rstd_out must be NULL.  Its backward is sp_region_bwd_exit.
 * x and gamma may not both be NULL. */
spr_status sp_region_fwd(const spr_desc* desc,
                         const void* x, const float* bias, const void* residual,
                         const float* gamma, const float* beta,
                         void* h_out, void* y_out, uint8_t* mask_out,
                         float* mean_out, float* rstd_out,
                         hipStream_t stream);

/* The forward with the reduce-scatter's arithmetic fused into its prologue.
 * Under sequence parallelism the row-parallel linear's partial outputs are
 * reduce-scattered instead of all-reduced, so rank i receives, for its own
 * tokens, the sum over the t ranks' partial outputs ("Tensor and sequence
 * parallelism -- explained with pictures", section "Add Sequence
 * parallelism"; "SP: Partition Activations Alongside TP", section "Connect
 * SP and TP across a layer").  This entry point takes those partial slabs
 * and sums them itself, so the reduced x is never written to or read from
 * memory:
 *  x_parts  [nparts][N][h] io   the partial slabs of this shard's rows, one
 *                               per rank in rank order (contiguous; slab p
 *                               at element offset p*N*h)
 *  nparts   1 .. 1024           (t for a direct reduce-scatter; 2 for the
 *                               last step of a ring)
 * x = round_io(x_parts[0] + x_parts[1] + ...): fp32 adds in rank order, one
 * rounding to the I/O type -- bit-identical to summing the slabs that way
 * and calling sp_region_fwd on the result.  Every other argument, check and
 * output is sp_region_fwd's; nparts = 1 is sp_region_fwd. */
spr_status sp_region_fwd_rs(const spr_desc* desc, const void* x_parts, int32_t nparts,
                            const float* bias, const void* residual,
                            const float* gamma, const float* beta,
                            void* h_out, void* y_out, uint8_t* mask_out,
                            float* mean_out, float* rstd_out,
                            hipStream_t stream);

/* Bytes of device workspace sp_region_bwd (and sp_region_bwd_exit) needs
 * for this desc on the current device: fp32 column partials of dgamma/
 * dbeta/dbias (one row of 3*h per row team, as many teams as the device has
 * compute units, or per row tile of the split path) and the split path's
 * per-row sums; or the exit's dbias partials (one row of h per 16-row
 * tile), whichever is larger.  0 on an invalid desc. */
size_t sp_region_bwd_workspace_bytes(const spr_desc* desc);

/* Backward of the region on one shard, from the forward's saved tensors.
 *  dy          [N,h] io   gradient of y
 *  dh_out      [N,h] io   gradient reaching h from outside the region (the
 *                         next block's residual branch); may be NULL (zero)
 *  h, mask, mean, rstd    as written by sp_region_fwd (mean is NULL for
 *                         RMSNorm; mask is NULL when p == 0, and with p > 0
 *                         NULL means: regenerate the forward's decisions
 *                         from desc's seed, offset, shard_index and t --
 *                         the desc must then be the forward's)
 *  gamma       [h]  fp32
 *  dx_out      [N,h] io   gradient of x; may be NULL (not written: the
 *                         norm-only entry has no x)
 *  dres_out    [N,h] io   gradient of residual (= gradient of h)
 *  dgamma_out  [h]  fp32  this shard's partial sum over its N rows
 *  dbeta_out   [h]  fp32  LayerNorm: required; RMSNorm: must be NULL
 *  dbias_out   [h]  fp32  may be NULL (not computed)
 *  workspace   device memory of at least sp_region_bwd_workspace_bytes,
 *              16-byte aligned; its contents on entry do not matter (every
 *              byte the call reads it writes first) and are undefined
 *              after.  Concurrent calls must use different workspaces.
 * The parameter gradients are this shard's partial sums; adding them over
 * the t shards (a tensor-parallel all-reduce) is the caller's.  The
 * reductions run in a fixed order: two identical calls give identical bits. */
spr_status sp_region_bwd(const spr_desc* desc,
                         const void* dy, const void* dh_out, const void* h,
                         const uint8_t* mask, const float* mean, const float* rstd,
                         const float* gamma,
                         void* dx_out, void* dres_out,
                         float* dgamma_out, float* dbeta_out, float* dbias_out,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* sp_region_bwd for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  The same arguments, checks, kernels and results (bit for bit)
 * as sp_region_bwd, without the workspace: its scratch is a fixed array of
 * SPR_NOALLOC_SCRATCH_BYTES in the library's device memory, one per GPU,
 * held from the first call on that GPU until the process ends.  The call
 * allocates nothing and frees nothing.
 *  - A desc whose backward needs more scratch than the array is
 *    SPR_ERR_WORKSPACE (checked before anything runs).  64 MiB covers every
 *    shard the fused path runs (h <= 12288 bf16: at most 256 partial rows of
 *    3*h fp32) and split-path shards of N rows with N * (8 + 3*h/8) bytes
 *    <= 64 MiB at the default 32-row tiles: [1024, 4, 25600] fits, the
 *    [2048, 4, 25600] shard (78.7 MB) does not.
 *  - Every call on one GPU uses that GPU's array: calls that may overlap on
 *    one GPU (two streams, or two host threads) race and give undefined
 *    results; serialise them, or use sp_region_bwd with one workspace each.
 *  - The array's contents on entry do not matter (the kernels write every
 *    byte they read first) and are left undefined. */
#define SPR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
spr_status sp_region_bwd_noalloc(const spr_desc* desc,
                                 const void* dy, const void* dh_out, const void* h,
                                 const uint8_t* mask, const float* mean, const float* rstd,
                                 const float* gamma,
                                 void* dx_out, void* dres_out,
                                 float* dgamma_out, float* dbeta_out, float* dbias_out,
                                 hipStream_t stream);

/* Backward of the norm-free exit (a forward with gamma == NULL):
 * dh = dh_out, so
 *  dh_out     [N,h] io   gradient of h (required)
 *  mask       as written by the forward (NULL when p == 0; with p > 0, NULL
 *             regenerates the decisions as in sp_region_bwd)
 *  dx_out     [N,h] io   keep ? dh_out * scale : 0
 *  dbias_out  [h]  fp32  this shard's partial sum of dx over its rows; may be
 *                        NULL (then no workspace is needed)
 *  workspace  at least sp_region_bwd_workspace_bytes(desc) bytes when
 *             dbias_out is given
 * The gradient of the residual is dh_out itself and is not written.  Same
 * conventions and checks as sp_region_bwd. */
spr_status sp_region_bwd_exit(const spr_desc* desc, const void* dh_out, const uint8_t* mask,
                              void* dx_out, float* dbias_out,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* The backward is a fixed sequence of kernel launches on `stream`: the row
 * pass(es), then a fixed-order column finalize of the parameter gradients.
 * sp_region_bwd runs the whole sequence.  These two let a caller run it one
 * launch at a time -- to time each kernel with events on the stream, or to
 * place the small finalize where it overlaps other work; launching indices
 * 0 .. n-1 in order on one stream is exactly sp_region_bwd.  Same arguments
 * and checks as sp_region_bwd.  sp_region_bwd_num_launches returns 0 for an
 * invalid desc; sp_region_bwd_launch returns SPR_ERR_INVALID_ARG for an
 * index outside 0 .. n-1. */
int sp_region_bwd_num_launches(const spr_desc* desc);
spr_status sp_region_bwd_launch(const spr_desc* desc, int index,
                                const void* dy, const void* dh_out, const void* h,
                                const uint8_t* mask, const float* mean, const float* rstd,
                                const float* gamma,
                                void* dx_out, void* dres_out,
                                float* dgamma_out, float* dbeta_out, float* dbias_out,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Bytes one forward call keeps (host arithmetic, no device access):
 *  saved_for_bwd   = h + mask (p > 0, stored) + per-token statistics
 *                    (a forward without a mask keeps N*h bytes fewer)
 *  retained_output = y, the next block's input
 * With bf16 I/O, a one-byte mask and two calls per layer (before attention
 * and before the MLP) this is 10*s*b*h/t bytes plus the statistics: the
 * replicated band of "Sequence parallel math" ("What tensor parallelism
 * leaves replicated"), divided by t. */
spr_status sp_region_activation_bytes(const spr_desc* desc, uint64_t* saved_for_bwd,
                                      uint64_t* retained_output);

/* Static description of a status code (any int; values that are no
 * spr_status give "unknown status"). */
const char* sp_region_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SP_REGION_H */
