/*
 * sp_oracle.c -- CPU oracle for the sequence-parallel (SP) region.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  Plain C, one
 * thread, one element at a time, written to be read against the pages rather
 * than to be fast.  It shares no code with the GPU library.
 *
 * Sources (cited by page title and section):
 *  - "Sequence parallel math" (transformer-math page on Megatron sequence
 *    parallelism): rank i owns tokens [i*s/t, (i+1)*s/t) ("The one-line
 *    idea"); LayerNorm normalises each token over the hidden dimension and
 *    residual dropout is elementwise, so a shard computes exactly the same
 *    result for its tokens ("The move: split the LayerNorm/dropout band along
 *    the sequence"); the band holds the two LayerNorm inputs, the two dropout
 *    masks and the block inputs, 10*s*b*h replicated under plain TP and
 *    10*s*b*h/t under SP ("What tensor parallelism leaves replicated", "The
 *    activation-memory saving, in one formula").
 *  - "Tensor and sequence parallelism -- explained with pictures", sections
 *    "Transformer block" (LayerNorm at the entrance of a sub-block, dropout on
 *    its output, residual from its input) and "Add Sequence parallelism"
 *    (reduce-scatter, then dropout locally, then the next sub-block).
 *  - "SP: Partition Activations Alongside TP", sections "Normalize and add
 *    residuals by token" (RMSNorm rescales one token from its own features;
 *    the residual has the same token layout) and "Connect SP and TP across a
 *    layer" (after reduce-scatter the SP region adds the residual and
 *    normalises again).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - order inside the region: h = residual + dropout(x + bias), y = Norm(h);
 *  - bias: an fp32 vector over h, added before dropout, optional;
 *  - inverted dropout: kept values are multiplied by scale = fp32(1/(1-p));
 *  - RNG: Philox4x32-10 (Salmon et al., SC'11), key = (seed lo, seed hi),
 *    counter = (e/4 lo, e/4 hi, offset lo, offset hi), element e uses output
 *    word e mod 4, where e is the element's flat index in the FULL [s, b, h]
 *    tensor, so every shard draws what the unsharded run would draw;
 *  - keep iff word >= floor(p * 2^32) (a tie keeps); p == 0 keeps all and
 *    writes no mask; the mask is one byte per element, 1 = keep;
 *  - h is rounded to the I/O type and the norm reads the rounded h;
 *  - LayerNorm: population variance, eps inside the square root;
 *    RMSNorm: y = gamma * h / sqrt(mean(h^2) + eps), no beta, no centring;
 *  - u, v and h are each one fp32 operation rounded to nearest even, with no
 *    fused multiply-add (this file is built with -ffp-contract=off); the
 *    statistics, y and every gradient are computed in float64 and rounded
 *    once at the end.
 */
#include "sp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10.  Multipliers and Weyl key increments as published by       */
/* Salmon et al. (SC'11) for the 4x32 variant.                                */
/* ------------------------------------------------------------------------ */
#define PHILOX_M4x32_0 0xD2511F53u
#define PHILOX_M4x32_1 0xCD9E8D57u
#define PHILOX_W32_0   0x9E3779B9u
#define PHILOX_W32_1   0xBB67AE85u

void spo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {               /* key schedule: bump between rounds */
            k0 += PHILOX_W32_0;
            k1 += PHILOX_W32_1;
        }
        uint64_t prod0 = (uint64_t)PHILOX_M4x32_0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)PHILOX_M4x32_1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

uint32_t spo_dropout_word(uint64_t seed, uint64_t offset, uint64_t e)
{
    uint64_t block = e / 4u;
    uint32_t ctr[4] = { (uint32_t)block, (uint32_t)(block >> 32),
                        (uint32_t)offset, (uint32_t)(offset >> 32) };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t out[4];
    spo_philox4x32_10(ctr, key, out);
    return out[e % 4u];
}

uint32_t spo_dropout_threshold(float p)
{
    /* p in [0,1): p * 2^32 is exact in double and below 2^32. */
    return (uint32_t)floor((double)p * 4294967296.0);
}

float spo_dropout_scale(float p)
{
    return (float)(1.0 / (1.0 - (double)p));
}

/* ------------------------------------------------------------------------ */
/* bfloat16: the upper 16 bits of an IEEE binary32.                           */
/* ------------------------------------------------------------------------ */
uint16_t spo_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);        /* NaN stays a quiet NaN */
    /* Round to nearest, ties to even, on the 16 discarded bits: add just under
     * half an ulp, plus one more when the kept lsb is odd. */
    uint32_t kept_lsb = (u >> 16) & 1u;
    u += 0x7fffu + kept_lsb;
    return (uint16_t)(u >> 16);
}

float spo_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------ */
/* I/O helpers                                                               */
/* ------------------------------------------------------------------------ */
static float load_io(int io, const void* base, int64_t i)
{
    if (io == SPO_BF16) return spo_bf16_to_f32(((const uint16_t*)base)[i]);
    return ((const float*)base)[i];
}

/* Rounds an fp32 value to the I/O type, stores it, and returns the stored
 * value widened back to fp32. */
static float store_io(int io, void* base, int64_t i, float v)
{
    if (io == SPO_BF16) {
        uint16_t b = spo_f32_to_bf16(v);
        ((uint16_t*)base)[i] = b;
        return spo_bf16_to_f32(b);
    }
    ((float*)base)[i] = v;
    return v;
}

static int desc_ok(const spo_desc* d)
{
    if (!d) return 0;
    if (d->s_local <= 0 || d->b <= 0 || d->h <= 0) return 0;
    if (d->t < 1 || d->shard_index < 0 || d->shard_index >= d->t) return 0;
    if (d->io != SPO_F32 && d->io != SPO_BF16) return 0;
    if (d->norm != SPO_LAYERNORM && d->norm != SPO_RMSNORM) return 0;
    if (!(d->p >= 0.0f && d->p < 1.0f)) return 0;
    if (!(d->eps > 0.0f)) return 0;
    return 1;
}

static int64_t rows_of(const spo_desc* d) { return d->s_local * d->b; }

/* Global flat index of (row r, column c) of this shard in the full tensor.
 * The shard is the contiguous slab starting at shard_index * N * h. */
static uint64_t global_elem(const spo_desc* d, int64_t r, int64_t c)
{
    uint64_t G = (uint64_t)d->shard_index * (uint64_t)rows_of(d) + (uint64_t)r;
    return G * (uint64_t)d->h + (uint64_t)c;
}

static int keep_elem(const spo_desc* d, int64_t r, int64_t c)
{
    if (d->p == 0.0f) return 1;
    uint32_t w = spo_dropout_word(d->seed, d->offset, global_elem(d, r, c));
    return w >= spo_dropout_threshold(d->p);
}

/* Per-token statistics of one row of the norm input, in float64, two-pass.
 * LayerNorm: mean and population variance; RMSNorm: mean square.
 * rstd = 1/sqrt(var + eps) or 1/sqrt(ms + eps). */
static void row_stats(const double* hrow, int64_t H, int norm, double eps,
                      double* mean, double* rstd)
{
    if (norm == SPO_LAYERNORM) {
        double sum = 0.0;
        for (int64_t c = 0; c < H; ++c) sum += hrow[c];
        double mu = sum / (double)H;
        double sq = 0.0;
        for (int64_t c = 0; c < H; ++c) sq += (hrow[c] - mu) * (hrow[c] - mu);
        double var = sq / (double)H;
        *mean = mu;
        *rstd = 1.0 / sqrt(var + eps);
    } else {
        double sq = 0.0;
        for (int64_t c = 0; c < H; ++c) sq += hrow[c] * hrow[c];
        double ms = sq / (double)H;
        *mean = 0.0;
        *rstd = 1.0 / sqrt(ms + eps);
    }
}

/* Backward through Norm for one row, in float64.
 *   xhat = (h - mean) * rstd         (RMSNorm: h * rstd)
 *   g    = dy * gamma
 *   LayerNorm: dh = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat))
 *   RMSNorm:   dh = rstd * (g - xhat * mean_c(g * xhat))
 * This is the chain rule through y = xhat * gamma (+ beta) with
 * d xhat_i / d h_j = rstd * (delta_ij - 1/H - xhat_i xhat_j / H) for
 * LayerNorm and rstd * (delta_ij - xhat_i xhat_j / H) for RMSNorm. */
static void norm_row_backward(int64_t H, int norm, double mean, double rstd,
                              const double* hrow, const double* dyrow,
                              const double* gam, double* xhat, double* dh)
{
    double sum_g = 0.0, sum_gx = 0.0;
    for (int64_t c = 0; c < H; ++c) {
        double xc = (norm == SPO_LAYERNORM) ? (hrow[c] - mean) * rstd : hrow[c] * rstd;
        double g = dyrow[c] * gam[c];
        xhat[c] = xc;
        sum_g += g;
        sum_gx += g * xc;
    }
    double mean_g = sum_g / (double)H, mean_gx = sum_gx / (double)H;
    for (int64_t c = 0; c < H; ++c) {
        double g = dyrow[c] * gam[c];
        if (norm == SPO_LAYERNORM)
            dh[c] = rstd * (g - mean_g - xhat[c] * mean_gx);
        else
            dh[c] = rstd * (g - xhat[c] * mean_gx);
    }
}

static int ptr_rules_fwd(const spo_desc* d, const void* beta, const void* mean_out,
                         const void* mask_out)
{
    if (d->norm == SPO_LAYERNORM && (!beta || !mean_out)) return 0;
    if (d->norm == SPO_RMSNORM && (beta || mean_out)) return 0;
    if (d->p > 0.0f && !mask_out) return 0;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Forward                                                                   */
/* ------------------------------------------------------------------------ */
/* Reduce-scatter prologue                                                   */
/* ------------------------------------------------------------------------ */
int spo_reduce_parts(const spo_desc* d, int nparts, const void* parts, void* x_out)
{
    if (!d || nparts < 1 || !parts || !x_out) return -1;
    const int64_t n = rows_of(d) * d->h;
    for (int64_t i = 0; i < n; ++i) {
        float acc = load_io(d->io, parts, i);                       /* rank 0 */
        for (int p = 1; p < nparts; ++p)
            acc = acc + load_io(d->io, parts, (int64_t)p * n + i);   /* fp32 add, rank order */
        store_io(d->io, x_out, i, acc);                              /* one rounding */
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
int spo_fwd(const spo_desc* d, int64_t r0, int64_t r1,
            const void* x, const float* bias, const void* residual,
            const float* gamma, const float* beta,
            void* h_out, void* y_out, uint8_t* mask_out,
            float* mean_out, float* rstd_out)
{
    if (!desc_ok(d)) return -1;
    const int64_t N = rows_of(d), H = d->h;
    if (r0 < 0 || r1 < r0 || r1 > N) return -1;
    if (!residual || (!x && !gamma)) return -1;
    if (x) {                                   /* the branch: x (+ bias), dropout */
        if (!h_out || (d->p > 0.0f && !mask_out)) return -1;
    } else {                                   /* norm-only entry: h is the residual */
        if (bias || mask_out || d->p > 0.0f) return -1;
    }
    if (gamma) {                               /* the norm */
        if (!y_out || !rstd_out) return -1;
        if (d->norm == SPO_LAYERNORM && (!beta || !mean_out)) return -1;
        if (d->norm == SPO_RMSNORM && (beta || mean_out)) return -1;
    } else {                                   /* norm-free exit */
        if (beta || y_out || mean_out || rstd_out) return -1;
    }

    const float scale = spo_dropout_scale(d->p);
    double* hrow = (double*)malloc((size_t)H * sizeof(double));
    if (!hrow) return -1;

    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t c = 0; c < H; ++c) {
            int64_t i = (r - r0) * H + c;
            if (!x) {                          /* no branch: h = residual, bit for bit */
                float hf = load_io(d->io, residual, i);
                hrow[c] = (double)(h_out ? store_io(d->io, h_out, i, hf) : hf);
                continue;
            }
            float u = load_io(d->io, x, i) + (bias ? bias[c] : 0.0f);   /* fp32 add */
            int keep = keep_elem(d, r, c);
            float v = keep ? u * scale : 0.0f;                          /* fp32 mul */
            float hf = load_io(d->io, residual, i) + v;                 /* fp32 add */
            hrow[c] = (double)store_io(d->io, h_out, i, hf);            /* norm reads rounded h */
            if (d->p > 0.0f) mask_out[i] = (uint8_t)keep;
        }
        if (!gamma) continue;
        double mu, rs;
        row_stats(hrow, H, d->norm, (double)d->eps, &mu, &rs);
        for (int64_t c = 0; c < H; ++c) {
            double yv;
            if (d->norm == SPO_LAYERNORM)
                yv = (hrow[c] - mu) * rs * (double)gamma[c] + (double)beta[c];
            else
                yv = hrow[c] * rs * (double)gamma[c];
            store_io(d->io, y_out, (r - r0) * H + c, (float)yv);
        }
        if (d->norm == SPO_LAYERNORM) mean_out[r - r0] = (float)mu;
        rstd_out[r - r0] = (float)rs;
    }
    free(hrow);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward                                                                  */
/* ------------------------------------------------------------------------ */
int spo_bwd(const spo_desc* d, int64_t r0, int64_t r1,
            const void* dy, const void* dh_out, const void* h,
            const uint8_t* mask, const float* mean, const float* rstd,
            const float* gamma,
            void* dx_out, void* dres_out,
            float* dgamma_out, float* dbeta_out, float* dbias_out)
{
    if (!desc_ok(d)) return -1;
    const int64_t N = rows_of(d), H = d->h;
    if (r0 < 0 || r1 < r0 || r1 > N) return -1;
    if (d->p > 0.0f && !mask) return -1;
    if (dy) {                                  /* through the norm */
        if (!h || !rstd || !gamma || !dres_out || !dgamma_out) return -1;
        if (d->norm == SPO_LAYERNORM && (!mean || !dbeta_out)) return -1;
        if (d->norm == SPO_RMSNORM && dbeta_out) return -1;
    } else {                                   /* norm-free exit: dh = dh_out */
        if (!dh_out || !dx_out || dgamma_out || dbeta_out) return -1;
    }

    const double scale = (double)spo_dropout_scale(d->p);
    double* buf = (double*)calloc((size_t)H * 8u, sizeof(double));
    if (!buf) return -1;
    double* hrow = buf;           double* dyrow = buf + H;     double* gam = buf + 2 * H;
    double* xhat = buf + 3 * H;   double* dh = buf + 4 * H;
    double* acc_dgamma = buf + 5 * H;  double* acc_dbeta = buf + 6 * H;
    double* acc_dbias = buf + 7 * H;

    if (dy)
        for (int64_t c = 0; c < H; ++c) gam[c] = (double)gamma[c];
    for (int64_t r = r0; r < r1; ++r) {
        if (dy) {
            for (int64_t c = 0; c < H; ++c) {
                hrow[c] = (double)load_io(d->io, h, (r - r0) * H + c);
                dyrow[c] = (double)load_io(d->io, dy, (r - r0) * H + c);
            }
            double mu = (d->norm == SPO_LAYERNORM) ? (double)mean[r - r0] : 0.0;
            norm_row_backward(H, d->norm, mu, (double)rstd[r - r0], hrow, dyrow, gam, xhat, dh);
        }
        for (int64_t c = 0; c < H; ++c) {
            int64_t i = (r - r0) * H + c;
            double dhv = (dy ? dh[c] : 0.0) + (dh_out ? (double)load_io(d->io, dh_out, i) : 0.0);
            int keep = (d->p > 0.0f) ? (mask[i] != 0) : 1;
            double dxu = keep ? dhv * scale : 0.0;
            if (dres_out) store_io(d->io, dres_out, i, (float)dhv);
            if (dx_out) store_io(d->io, dx_out, i, (float)dxu);
            if (dy) {
                acc_dgamma[c] += dyrow[c] * xhat[c];
                acc_dbeta[c] += dyrow[c];
            }
            acc_dbias[c] += dxu;
        }
    }
    for (int64_t c = 0; c < H; ++c) {
        if (dgamma_out) dgamma_out[c] = (float)acc_dgamma[c];
        if (dbeta_out) dbeta_out[c] = (float)acc_dbeta[c];
        if (dbias_out) dbias_out[c] = (float)acc_dbias[c];
    }
    free(buf);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* All-float64 forms (finite-difference checks)                              */
/* ------------------------------------------------------------------------ */
int spo_fwd_exact(const spo_desc* d, const double* x, const double* bias,
                  const double* residual, const double* gamma, const double* beta,
                  double* h_out, double* y_out, uint8_t* mask_out,
                  double* mean_out, double* rstd_out)
{
    if (!desc_ok(d)) return -1;
    if (!x || !residual || !gamma || !h_out || !y_out || !rstd_out) return -1;
    if (!ptr_rules_fwd(d, beta, mean_out, mask_out)) return -1;
    const int64_t N = rows_of(d), H = d->h;
    const double scale = (double)spo_dropout_scale(d->p);
    for (int64_t r = 0; r < N; ++r) {
        for (int64_t c = 0; c < H; ++c) {
            int64_t i = r * H + c;
            double u = x[i] + (bias ? bias[c] : 0.0);
            int keep = keep_elem(d, r, c);
            h_out[i] = residual[i] + (keep ? u * scale : 0.0);
            if (d->p > 0.0f) mask_out[i] = (uint8_t)keep;
        }
        double mu, rs;
        row_stats(h_out + r * H, H, d->norm, (double)d->eps, &mu, &rs);
        for (int64_t c = 0; c < H; ++c) {
            int64_t i = r * H + c;
            y_out[i] = (d->norm == SPO_LAYERNORM) ? (h_out[i] - mu) * rs * gamma[c] + beta[c]
                                                  : h_out[i] * rs * gamma[c];
        }
        if (d->norm == SPO_LAYERNORM) mean_out[r] = mu;
        rstd_out[r] = rs;
    }
    return 0;
}

int spo_bwd_exact(const spo_desc* d, const double* dy, const double* dh_out,
                  const double* h, const uint8_t* mask,
                  const double* mean, const double* rstd, const double* gamma,
                  double* dx_out, double* dres_out,
                  double* dgamma_out, double* dbeta_out, double* dbias_out)
{
    if (!desc_ok(d)) return -1;
    if (!dy || !h || !rstd || !gamma || !dx_out || !dres_out || !dgamma_out) return -1;
    if (d->norm == SPO_LAYERNORM && (!mean || !dbeta_out)) return -1;
    if (d->norm == SPO_RMSNORM && dbeta_out) return -1;
    if (d->p > 0.0f && !mask) return -1;
    const int64_t N = rows_of(d), H = d->h;
    const double scale = (double)spo_dropout_scale(d->p);
    double* buf = (double*)malloc((size_t)H * 2u * sizeof(double));
    if (!buf) return -1;
    double* xhat = buf; double* dh = buf + H;
    for (int64_t c = 0; c < H; ++c) {
        dgamma_out[c] = 0.0;
        if (dbeta_out) dbeta_out[c] = 0.0;
        if (dbias_out) dbias_out[c] = 0.0;
    }
    for (int64_t r = 0; r < N; ++r) {
        double mu = (d->norm == SPO_LAYERNORM) ? mean[r] : 0.0;
        norm_row_backward(H, d->norm, mu, rstd[r], h + r * H, dy + r * H, gamma, xhat, dh);
        for (int64_t c = 0; c < H; ++c) {
            int64_t i = r * H + c;
            double dhv = dh[c] + (dh_out ? dh_out[i] : 0.0);
            int keep = (d->p > 0.0f) ? (mask[i] != 0) : 1;
            double dxu = keep ? dhv * scale : 0.0;
            dres_out[i] = dhv;
            dx_out[i] = dxu;
            dgamma_out[c] += dy[i] * xhat[c];
            if (dbeta_out) dbeta_out[c] += dy[i];
            if (dbias_out) dbias_out[c] += dxu;
        }
    }
    free(buf);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Accounting                                                                */
/* ------------------------------------------------------------------------ */
int spo_activation_bytes(const spo_desc* d, uint64_t* saved_for_bwd,
                         uint64_t* retained_output)
{
    if (!desc_ok(d) || !saved_for_bwd || !retained_output) return -1;
    uint64_t N = (uint64_t)rows_of(d), E = N * (uint64_t)d->h;
    uint64_t es = (d->io == SPO_BF16) ? 2u : 4u;
    uint64_t mask_bytes = (d->p > 0.0f) ? E : 0u;           /* one byte per element  */
    uint64_t stat_bytes = N * ((d->norm == SPO_LAYERNORM) ? 8u : 4u);  /* fp32 mean, rstd */
    *saved_for_bwd = E * es + mask_bytes + stat_bytes;       /* h (the norm input) + mask + stats */
    *retained_output = E * es;                               /* y, the next block's input */
    return 0;
}

void spo_layer_activation_elems(double s, double b, double h, double a, double t,
                                double* full, double* tp, double* tp_sp)
{
    double sbh = s * b * h;
    *full = sbh * (34.0 + 5.0 * a * s / h);
    *tp = sbh * (10.0 + 24.0 / t + 5.0 * a * s / (h * t));
    *tp_sp = sbh / t * (34.0 + 5.0 * a * s / h);
}

/* ------------------------------------------------------------------------ */
/* Ring attention: ordinary attention over all keys (see the header)         */
/* ------------------------------------------------------------------------ */
int spo_attention(const spo_attn_desc* d, int64_t r0, int64_t r1, const uint16_t* q,
                  const uint16_t* k, const uint16_t* v, double* o_out, double* lse_out)
{
    if (!d || !q || !k || !v || !o_out || !lse_out) return -1;
    if (r0 < 0 || r1 < r0 || r1 > d->s_local) return -1;
    if (d->s_local < 1 || d->b < 1 || d->heads < 1 || d->d < 1 || d->t < 1) return -1;
    if (d->rank < 0 || d->rank >= d->t || !(d->scale > 0.0f)) return -1;
    const int64_t S = d->s_local, B = d->b, NH = d->heads, D = d->d;
    const int64_t nkeys = (int64_t)d->t * S;               /* keys per (batch, head) */
    double* s = (double*)malloc((size_t)nkeys * sizeof(double));
    if (!s) return -1;
    /* element (token, batch, head, dim) of a [tokens][b][heads][d] tensor */
#define AT(tok, bi, hh, dd) ((((tok) * B + (bi)) * NH + (hh)) * D + (dd))
    for (int64_t qi = 0; qi < r1 - r0; ++qi)                    /* query token r0 + qi */
        for (int64_t bi = 0; bi < B; ++bi)
            for (int64_t hh = 0; hh < NH; ++hh) {
                double m = -INFINITY;
                for (int64_t j = 0; j < nkeys; ++j) {           /* key token j of the sequence */
                    double dot = 0.0;
                    for (int64_t dd = 0; dd < D; ++dd)
                        dot += (double)spo_bf16_to_f32(q[AT(qi, bi, hh, dd)]) *
                               (double)spo_bf16_to_f32(k[AT(j, bi, hh, dd)]);
                    s[j] = (double)d->scale * dot;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < nkeys; ++j) l += exp(s[j] - m);
                for (int64_t dd = 0; dd < D; ++dd) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < nkeys; ++j)
                        acc += exp(s[j] - m) * (double)spo_bf16_to_f32(v[AT(j, bi, hh, dd)]);
                    o_out[AT(qi, bi, hh, dd)] = acc / l;
                }
                lse_out[(qi * B + bi) * NH + hh] = m + log(l);
            }
#undef AT
    free(s);
    return 0;
}
