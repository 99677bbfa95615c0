/*
 * sp_oracle.h -- CPU oracle for the sequence-parallel (SP) region.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the GPU
 * library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or constant with the GPU library.
 *
 * What it computes (one rank's token shard [s/t, b, h], sequence-major):
 *   forward   u = x + bias ; v = dropout(u) ; h = residual + v ; y = Norm(h)
 *   backward  dx, dresidual, dgamma, dbeta, dbias for that composition.
 * The region is the LayerNorm/dropout/residual band that sequence parallelism
 * splits along the sequence ("Sequence parallel math", sections "The one-line
 * idea" and "The move: split the LayerNorm/dropout band along the sequence";
 * "Tensor and sequence parallelism -- explained with pictures", section "Add
 * Sequence parallelism"; "SP: Partition Activations Alongside TP", sections
 * "Normalize and add residuals by token" and "Connect SP and TP across a
 * layer").
 *
 * Parity status of every function is stated at its declaration.
 */
#ifndef SP_ORACLE_H
#define SP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* I/O element type of x, residual, h, y, dy, dh_out, dx, dresidual.
 * bf16 values travel as their raw 16-bit patterns (uint16_t). */
enum { SPO_F32 = 0, SPO_BF16 = 1 };
/* Normalisation: LayerNorm (centre + scale + beta) or RMSNorm (scale only). */
enum { SPO_LAYERNORM = 0, SPO_RMSNORM = 1 };

typedef struct {
    int64_t  s_local;      /* tokens of this shard along the sequence (s/t)      */
    int64_t  b;            /* batch                                              */
    int64_t  h;            /* hidden size                                        */
    int32_t  shard_index;  /* rank i owns tokens [i*s/t, (i+1)*s/t)              */
    int32_t  t;            /* sequence/tensor-parallel degree                    */
    int32_t  io;           /* SPO_F32 or SPO_BF16                                */
    int32_t  norm;         /* SPO_LAYERNORM or SPO_RMSNORM                       */
    float    p;            /* dropout probability, 0 <= p < 1                    */
    float    eps;          /* added to the variance / mean square, > 0           */
    uint64_t seed;         /* Philox key                                         */
    uint64_t offset;       /* Philox stream (e.g. one per dropout site)          */
} spo_desc;

/* Philox4x32-10 block function (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11).  Pinned against an independent
 * library implementation of the same generator. */
void spo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The 32-bit word that decides element e (global flat index of the full
 * [s, b, h] tensor) for dropout site (seed, offset). */
uint32_t spo_dropout_word(uint64_t seed, uint64_t offset, uint64_t e);

/* Drop threshold floor(p * 2^32) and inverted-dropout scale 1/(1-p) (fp32). */
uint32_t spo_dropout_threshold(float p);
float    spo_dropout_scale(float p);

/* float -> bfloat16 round-to-nearest-even and the exact widening back.
 * Pinned against torch's float32 -> bfloat16 conversion. */
uint16_t spo_f32_to_bf16(float f);
float    spo_bf16_to_f32(uint16_t b);

/* Reduce-scatter prologue of the region: x = round_io(sum over p of
 * parts[p]) for every element of the shard, the parts added in rank order
 * p = 0, 1, ..., nparts-1, each add one fp32 operation, then one rounding to
 * the I/O type.  parts is [nparts][N][h] and x_out [N][h], both in the I/O
 * type (N = s_local*b).  After the row-parallel linear each rank holds a
 * partial sum of the block's output; the reduce-scatter that replaces the
 * all-reduce under sequence parallelism hands rank i the sum over ranks of
 * its own tokens' rows ("Tensor and sequence parallelism -- explained with
 * pictures", section "Add Sequence parallelism"; "SP: Partition Activations
 * Alongside TP", section "Connect SP and TP across a layer").  The order and
 * the single rounding are this library's reading.  Returns 0, or -1 for
 * nparts < 1 or a NULL pointer.
 * Parity: pinned (identity at nparts = 1, exact integer sums, a case whose
 * result depends on the order, bf16 ties of the final rounding). */
int spo_reduce_parts(const spo_desc* d, int nparts, const void* parts, void* x_out);

/* Forward over rows [r0, r1) of the shard.  Every per-row array (x, residual,
 * h_out, y_out, mask_out, mean_out, rstd_out) starts at row r0: element (r, c)
 * lives at index (r - r0) * h + c, and r only enters the global index.
 * bias may be NULL (the same as a zero bias: u = x + 0.0f).  beta and
 * mean_out must be NULL for RMSNorm.  mask_out is not written when p == 0 (may be NULL).
 * Two variants at the ends of the layer stack (a block boundary with no
 * branch before the first LayerNorm, and none after the last residual add):
 *  - x == NULL, the norm-only entry: no branch, h is the residual bit for
 *    bit (no add), y = Norm(residual); p must be 0, bias and mask_out NULL,
 *    h_out may be NULL (then h is not written);
 *  - gamma == NULL, the norm-free exit: h and the mask only; beta, y_out,
 *    mean_out and rstd_out must be NULL.
 * Returns 0 on success, -1 on an invalid argument.
 * Pinned: p=0 identity, dropout expectation, LayerNorm/RMSNorm closed forms,
 * float64 torch layer_norm / rms_norm, shard invariance. */
int spo_fwd(const spo_desc* d, int64_t r0, int64_t r1,
            const void* x, const float* bias, const void* residual,
            const float* gamma, const float* beta,
            void* h_out, void* y_out, uint8_t* mask_out,
            float* mean_out, float* rstd_out);

/* Backward over rows [r0, r1); per-row arrays start at row r0 as above.
 * Uses the stored h, mask, mean and rstd of the forward.  dh_out (gradient reaching h from elsewhere, e.g. the next block's
 * residual branch) may be NULL.  dgamma/dbeta/dbias receive the partial sums
 * over rows [r0, r1) (fp32); dbeta must be NULL for RMSNorm; dbias may be
 * NULL.  mask may be NULL when p == 0.  dx_out may be NULL (not written:
 * the norm-only entry has no branch).  dy == NULL is the norm-free exit:
 * dh = dh_out (required), h, mean, rstd and gamma are not read,
 * dgamma_out and dbeta_out must be NULL, dres_out may be NULL.
 * Pinned: central finite differences of spo_fwd_exact, float64 torch
 * autograd, the per-row identity sum_c dh = 0 for LayerNorm. */
int spo_bwd(const spo_desc* d, int64_t r0, int64_t r1,
            const void* dy, const void* dh_out, const void* h,
            const uint8_t* mask, const float* mean, const float* rstd,
            const float* gamma,
            void* dx_out, void* dres_out,
            float* dgamma_out, float* dbeta_out, float* dbias_out);

/* All-float64 forms of the same computation, with no rounding to the I/O
 * type anywhere (the mask still comes from Philox).  Used to take finite
 * differences.  Same argument rules as above; d->io is ignored. */
int spo_fwd_exact(const spo_desc* d, const double* x, const double* bias,
                  const double* residual, const double* gamma, const double* beta,
                  double* h_out, double* y_out, uint8_t* mask_out,
                  double* mean_out, double* rstd_out);
int spo_bwd_exact(const spo_desc* d, const double* dy, const double* dh_out,
                  const double* h, const uint8_t* mask,
                  const double* mean, const double* rstd, const double* gamma,
                  double* dx_out, double* dres_out,
                  double* dgamma_out, double* dbeta_out, double* dbias_out);

/* Bytes one call keeps: saved_for_bwd = h + mask + per-token stats,
 * retained_output = y (the next block's input).  Two calls per layer give
 * the replicated band of "Sequence parallel math", section "What tensor
 * parallelism leaves replicated", divided by t.  Pinned by that page's
 * figures (tests/golden). */
int spo_activation_bytes(const spo_desc* d, uint64_t* saved_for_bwd,
                         uint64_t* retained_output);

/* The per-layer activation model of "Sequence parallel math", sections "The
 * problem: activation memory, not weight memory" and "The activation-memory
 * saving, in one formula", in elements:
 *   full   = s*b*h*(34 + 5*a*s/h)
 *   tp     = s*b*h*(10 + 24/t + 5*a*s/(h*t))
 *   tp_sp  = s*b*h/t*(34 + 5*a*s/h)
 * Pinned by the page's worked numeric example (tests/golden). */
void spo_layer_activation_elems(double s, double b, double h, double a, double t,
                                double* full, double* tp, double* tp_sp);

/* ------------------------------------------------------------------------
 * Ring attention (context parallelism), one rank's forward.
 *
 * Context parallelism shards Q, K and V along the sequence: rank i owns a
 * contiguous block of query tokens and the matching K/V block.  Ring
 * attention passes the K/V blocks around the ring; at each step a rank
 * attends its queries to the block in hand and accumulates the partial
 * online-softmax result, and after t steps every query has attended every
 * key ("Sequence parallel math", section "Context parallelism and ring
 * attention").  The pages apply no causal mask: every query sees every key.
 * Whatever the order of the steps, the result is ordinary attention of the
 * rank's queries over the whole sequence, which is what this function
 * computes, in float64, straight from the definition:
 *   s_j = scale * (q . k_j),  o = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),
 *   lse = m + log(sum_j exp(s_j - m)),  m = max_j s_j,
 * over the keys j of all t blocks with the query's batch index and head.
 * Layouts (bf16 as raw 16-bit words): q [s_local][b][heads][d]; k and v
 * [t][s_local][b][heads][d] (block j = the tokens of rank j); o_out
 * [s_local][b][heads][d] and lse_out [s_local][b][heads] in float64.  Only
 * the rank's query tokens [r0, r1) are computed: q, o_out and lse_out start
 * at token r0 (as the region's row ranges).  rank does not change the result
 * (it orders the ring).  Returns 0, or -1 on an invalid argument.
 * Parity: pinned (torch float64 scaled_dot_product_attention, a single key,
 * identical keys, constant values, a two-key closed form, invariance to the
 * order of the key blocks). */
typedef struct {
    int64_t s_local;   /* query tokens of this rank = key tokens per block */
    int64_t b;         /* batch                                            */
    int32_t heads;     /* attention heads                                  */
    int32_t d;         /* head dimension                                   */
    int32_t t;         /* ring size (context-parallel degree)              */
    int32_t rank;      /* this rank (owns query block `rank`)              */
    float   scale;     /* softmax scale, usually 1/sqrt(d)                 */
} spo_attn_desc;

int spo_attention(const spo_attn_desc* d, int64_t r0, int64_t r1, const uint16_t* q,
                  const uint16_t* k, const uint16_t* v, double* o_out, double* lse_out);

#ifdef __cplusplus
}
#endif
#endif /* SP_ORACLE_H */
