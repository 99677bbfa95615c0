// sp_bwd.hip -- backward of the sequence-parallel region on gfx950.
//
// Chain rule through y = Norm(h) * gamma (+ beta), h = residual + dropout(x + bias):
//   xhat = (h - mean) * rstd            (RMSNorm: h * rstd)
//   g    = dy * gamma
//   dh   = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat)) + dh_out
//          (RMSNorm drops the mean_c(g) term)
//   dresidual = dh,  dx = keep ? dh * scale : 0
//   dgamma = sum_r dy * xhat,  dbeta = sum_r dy,  dbias = sum_r dx
// The pages only say that the band's activations are kept for the backward
// ("Sequence parallel math", section "The one-line idea"); the formulas are
// the derivative of the forward.
//
// Kernel 1 (row teams): each team walks rows r = team, team + teams, ...;
// a row's two sums are one team reduction, dx/dresidual are written once,
// and the thread's columns accumulate dgamma/dbeta/dbias partials in
// registers.  Each team writes one fp32 partial row of 3*h.
// Kernel 2 (finalize): per column, the partial rows are added in team order,
// so the result does not depend on scheduling.
#include "sp_device.h"
#include "sp_plan.h"

namespace spr {

template <typename IO, int NORM, bool DROP, int VPT, bool WAVE_ROWS, int LB>
__global__ void __launch_bounds__(LB) sp_region_bwd_rows_kernel(BwdArgs a) {
    using V = Vec<IO>;
    constexpr int E = V::N;
    __shared__ float red[2][32];

    int tid, tpr, nwaves;
    int64_t team;
    if (WAVE_ROWS) {
        tid = threadIdx.x & 63;
        tpr = 64;
        nwaves = 1;
        team = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    } else {
        tid = threadIdx.x;
        tpr = blockDim.x;
        nwaves = blockDim.x >> 6;
        team = blockIdx.x;
    }

    float acc_g[VPT][E], acc_b[VPT][E], acc_x[VPT][E];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
        for (int j = 0; j < E; ++j) acc_g[k][j] = acc_b[k][j] = acc_x[k][j] = 0.0f;
    }

    int slot = 0;
    // The trip count is uniform over the team (and over the workgroup when
    // the workgroup is the team), so every thread meets every barrier.
    for (int64_t row = team; row < a.rows; row += a.teams) {
        const int64_t rbase = row * a.hidden;
        V hv[VPT], dyv[VPT];
        uint32_t kb[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int vec = k * tpr + tid;
            kb[k] = 0xffu;
            if (vec < a.nvec) {
                const int64_t off = rbase + (int64_t)vec * E;
                hv[k].load(static_cast<const IO*>(a.h) + off);
                dyv[k].load(static_cast<const IO*>(a.dy) + off);
                if (DROP) kb[k] = MaskBytes<E>::load(a.mask + off);
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) hv[k].v[j] = dyv[k].v[j] = 0.0f;
            }
        }
        const float mu = (NORM == SPR_LAYERNORM) ? a.mean[row] : 0.0f;
        const float rs = a.rstd[row];

        // g and xhat are recomputed in the second pass rather than kept
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int vec = k * tpr + tid;
            if (vec < a.nvec) {
                float gam[E];
                load_params<E>(a.gamma + (int64_t)vec * E, gam);
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const float xh = (hv[k].v[j] - mu) * rs;
                    const float g = dyv[k].v[j] * gam[j];
                    s1 += g;
                    s2 += g * xh;
                }
            }
        }
        block_sum2(s1, s2, red[slot], nwaves);
        slot ^= 1;
        const float mg = s1 * a.inv_h, mgx = s2 * a.inv_h;

#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int vec = k * tpr + tid;
            if (vec < a.nvec) {
                const int64_t off = rbase + (int64_t)vec * E;
                V dho;
                if (a.dh_out) dho.load(static_cast<const IO*>(a.dh_out) + off);
                float gam[E];
                load_params<E>(a.gamma + (int64_t)vec * E, gam);
                V dres, dx;
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const float xh = (hv[k].v[j] - mu) * rs;
                    const float g = dyv[k].v[j] * gam[j];
                    float dh = (NORM == SPR_LAYERNORM) ? rs * (g - mg - xh * mgx)
                                                       : rs * (g - xh * mgx);
                    if (a.dh_out) dh += dho.v[j];
                    const float dxu = DROP ? (((kb[k] >> j) & 1u) ? dh * a.scale : 0.0f) : dh;
                    dres.v[j] = dh;
                    dx.v[j] = dxu;
                    acc_g[k][j] += dyv[k].v[j] * xh;
                    acc_b[k][j] += dyv[k].v[j];
                    acc_x[k][j] += dxu;
                }
                dres.store(static_cast<IO*>(a.dres_out) + off);
                dx.store(static_cast<IO*>(a.dx_out) + off);
            }
        }
    }

    float* part = a.partials + team * 3 * a.hidden;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        if (vec < a.nvec) {
            const int64_t c = (int64_t)vec * E;
#pragma unroll
            for (int j = 0; j < E; j += 4) {
                *reinterpret_cast<float4*>(part + c + j) =
                    make_float4(acc_g[k][j], acc_g[k][j + 1], acc_g[k][j + 2], acc_g[k][j + 3]);
                *reinterpret_cast<float4*>(part + a.hidden + c + j) =
                    make_float4(acc_b[k][j], acc_b[k][j + 1], acc_b[k][j + 2], acc_b[k][j + 3]);
                *reinterpret_cast<float4*>(part + 2 * a.hidden + c + j) =
                    make_float4(acc_x[k][j], acc_x[k][j + 1], acc_x[k][j + 2], acc_x[k][j + 3]);
            }
        }
    }
}

// out_k[c] = sum over teams t (in order) of partials[t][k][c], k = dgamma,
// dbeta, dbias; an output whose pointer is NULL is skipped.
__global__ void __launch_bounds__(256) sp_region_bwd_finalize_kernel(BwdArgs a) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= 3 * a.hidden) return;
    const int k = (int)(j / a.hidden);
    const int64_t c = j - (int64_t)k * a.hidden;
    float* out = k == 0 ? a.dgamma_out : (k == 1 ? a.dbeta_out : a.dbias_out);
    if (!out) return;
    const float* p = a.partials + (int64_t)k * a.hidden + c;
    float s = 0.0f;
    for (int t = 0; t < a.teams; ++t) s += p[(int64_t)t * 3 * a.hidden];
    out[c] = s;
}

// Teams: enough to cover the chip a couple of times over while keeping the
// partial rows (3*h fp32 each, written once and read once) few.
int64_t bwd_teams(const spr_desc& d, const RowPlan& p) {
    const int64_t rows = d.s_local * d.b;
    const int64_t cap = 256;
    const int64_t want = rows < cap ? rows : cap;
    return ((want + p.rpw - 1) / p.rpw) * p.rpw;
}

template <typename IO, int NORM, bool DROP, bool WR>
static hipError_t bwd_by_vpt(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    const dim3 g((unsigned)(a.teams / p.rpw)), b((unsigned)p.block);
#define SPR_BWD_CASE(V, L)                                                                       \
    case V:                                                                                      \
        hipLaunchKernelGGL((sp_region_bwd_rows_kernel<IO, NORM, DROP, V, WR, L>), g, b, 0, s, a); \
        break;
    if (WR) {
        switch (p.vpt) {
            SPR_BWD_CASE(1, 256) SPR_BWD_CASE(2, 256) SPR_BWD_CASE(3, 256) SPR_BWD_CASE(4, 256)
            default: return hipErrorInvalidValue;
        }
    } else {
        // must match kWgCombos
        switch (p.vpt) {
            SPR_BWD_CASE(1, 1024) SPR_BWD_CASE(2, 1024) SPR_BWD_CASE(3, 1024)
            SPR_BWD_CASE(4, 1024) SPR_BWD_CASE(5, 768) SPR_BWD_CASE(6, 768) SPR_BWD_CASE(8, 512)
            default: return hipErrorInvalidValue;
        }
    }
#undef SPR_BWD_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = 3 * a.hidden;
    hipLaunchKernelGGL(sp_region_bwd_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                       0, s, a);
    return hipGetLastError();
}

template <typename IO, int NORM, bool DROP>
static hipError_t bwd_by_mode(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    return p.rpw > 1 ? bwd_by_vpt<IO, NORM, DROP, true>(p, a, s)
                     : bwd_by_vpt<IO, NORM, DROP, false>(p, a, s);
}

template <typename IO, int NORM>
static hipError_t bwd_by_drop(const spr_desc& d, const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    return d.p > 0.0f ? bwd_by_mode<IO, NORM, true>(p, a, s) : bwd_by_mode<IO, NORM, false>(p, a, s);
}

template <typename IO>
static hipError_t bwd_by_norm(const spr_desc& d, const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    return d.norm == SPR_LAYERNORM ? bwd_by_drop<IO, SPR_LAYERNORM>(d, p, a, s)
                                   : bwd_by_drop<IO, SPR_RMSNORM>(d, p, a, s);
}

hipError_t launch_bwd(const spr_desc& d, const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    return d.io == SPR_BF16 ? bwd_by_norm<__bf16>(d, p, a, s) : bwd_by_norm<float>(d, p, a, s);
}

}  // namespace spr
