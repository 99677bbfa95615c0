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

// The saved tensors of one row as loaded (raw words; decoded when used).
template <int VPT, int MW>
struct RowIn {
    uint4 h[VPT], dy[VPT], dho[VPT];
    uint32_t mask[VPT][MW];
    float mu, rs;
};

template <typename IO, int NORM, bool DROP, int VPT, bool WAVE_ROWS, int LB>
__global__ void __launch_bounds__(LB) sp_region_bwd_rows_kernel(BwdArgs a) {
    // Prefetching the next row doubles the row's registers; wide rows
    // (more than two vectors per thread) load each row when they reach it.
    constexpr bool PREFETCH = VPT <= 2;
    using V = Vec<IO>;
    constexpr int E = V::N;
    constexpr int MW = E / 4;                 // mask words per vector
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

    // Idle vector slots of a ragged row re-read the row's last vector; their
    // results are masked out of every sum and never stored.
    int vc[VPT];
    bool ok[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        ok[k] = vec < a.nvec;
        vc[k] = ok[k] ? vec : a.nvec - 1;
    }

    float gam[VPT][E], acc_g[VPT][E], acc_b[VPT][E], acc_x[VPT][E];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        load_params<E>(a.gamma + (int64_t)vc[k] * E, gam[k]);
#pragma unroll
        for (int j = 0; j < E; ++j) acc_g[k][j] = acc_b[k][j] = acc_x[k][j] = 0.0f;
    }

    auto load_row = [&](int64_t row, RowIn<VPT, MW>& in) {
        const int64_t rbase = row * a.hidden;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int64_t off = rbase + (int64_t)vc[k] * E;
            in.h[k] = load_stream(static_cast<const IO*>(a.h) + off);
            in.dy[k] = load_stream(static_cast<const IO*>(a.dy) + off);
            if (DROP) {
#pragma unroll
                for (int w = 0; w < MW; ++w)
                    in.mask[k][w] = __builtin_nontemporal_load(
                        reinterpret_cast<const uint32_t*>(a.mask + off) + w);
            }
            if (a.dh_out) in.dho[k] = load_stream(static_cast<const IO*>(a.dh_out) + off);
        }
        in.mu = (NORM == SPR_LAYERNORM) ? a.mean[row] : 0.0f;
        in.rs = a.rstd[row];
    };

    // Rows team, team + teams, ...: the trip count is uniform over the team
    // (the workgroup, when the workgroup is the team), so every thread meets
    // every barrier.  The next row's loads are issued before this row's
    // reduction, so they are in flight while it is computed and stored.
    RowIn<VPT, MW> cur, nxt;
    int64_t row = team;
    if (PREFETCH && row < a.rows) load_row(row, cur);
    int slot = 0;
    for (; row < a.rows; row += a.teams) {
        const int64_t next = row + a.teams;
        if (PREFETCH) {
            if (next < a.rows) load_row(next, nxt);
        } else {
            load_row(row, cur);
        }

        V hv[VPT], dyv[VPT];
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            hv[k].set(cur.h[k]);
            dyv[k].set(cur.dy[k]);
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float xh = (hv[k].v[j] - cur.mu) * cur.rs;
                const float g = dyv[k].v[j] * gam[k][j];
                if (ok[k]) {
                    s1 += g;
                    s2 += g * xh;
                }
            }
        }
        block_sum2(s1, s2, red[slot], nwaves);
        slot ^= 1;
        const float mg = s1 * a.inv_h, mgx = s2 * a.inv_h;

        const int64_t rbase = row * a.hidden;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            V dho, dres, dx;
            if (a.dh_out) dho.set(cur.dho[k]);
            uint32_t kb = 0xffu;
            if (DROP) {
                kb = MaskBytes<4>::from_word(cur.mask[k][0]);
                if (MW == 2) kb |= MaskBytes<4>::from_word(cur.mask[k][MW - 1]) << 4;
            }
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float xh = (hv[k].v[j] - cur.mu) * cur.rs;
                const float g = dyv[k].v[j] * gam[k][j];
                float dh = (NORM == SPR_LAYERNORM) ? cur.rs * (g - mg - xh * mgx)
                                                   : cur.rs * (g - xh * mgx);
                if (a.dh_out) dh += dho.v[j];
                const float dxu = DROP ? (((kb >> j) & 1u) ? dh * a.scale : 0.0f) : dh;
                dres.v[j] = dh;
                dx.v[j] = dxu;
                if (ok[k]) {
                    acc_g[k][j] += dyv[k].v[j] * xh;
                    acc_b[k][j] += dyv[k].v[j];
                    acc_x[k][j] += dxu;
                }
            }
            if (ok[k]) {
                const int64_t off = rbase + (int64_t)vc[k] * E;
                dres.store(static_cast<IO*>(a.dres_out) + off);
                dx.store(static_cast<IO*>(a.dx_out) + off);
            }
        }
        if (PREFETCH) cur = nxt;
    }

    float* part = a.partials + team * 3 * a.hidden;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (ok[k]) {
            const int64_t c = (int64_t)vc[k] * E;
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

// out_k[c] = sum over teams t = 0, 1, ... of partials[t][k][c] (k = dgamma,
// dbeta, dbias over the flat index j = k*h + c).  A workgroup owns 64
// consecutive j (16 lanes x float4) and splits the teams over 16 lane
// groups: group q adds teams q, q+16, ... in order, then the 16 group sums
// are added in group order.  Fixed order throughout: the result does not
// depend on scheduling.  An output whose pointer is NULL is skipped.
constexpr int kFinCols = 64, kFinGroups = 16;
__global__ void __launch_bounds__(256) sp_region_bwd_finalize_kernel(BwdArgs a) {
    __shared__ float4 part[kFinGroups][kFinCols / 4];
    const int lane = threadIdx.x % (kFinCols / 4), q = threadIdx.x / (kFinCols / 4);
    const int64_t j = (int64_t)blockIdx.x * kFinCols + lane * 4;
    const int64_t n3 = 3 * a.hidden;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j < n3) {
        const float* p = a.partials + j;
        for (int t = q; t < a.teams; t += kFinGroups) {
            const float4 v = *reinterpret_cast<const float4*>(p + (int64_t)t * n3);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
    }
    part[q][lane] = s;
    __syncthreads();
    if (q == 0 && j < n3) {
        float4 t = part[0][lane];
        for (int g = 1; g < kFinGroups; ++g) {
            const float4 v = part[g][lane];
            t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
        }
        const int k = (int)(j / a.hidden);
        const int64_t c = j - (int64_t)k * a.hidden;
        float* out = k == 0 ? a.dgamma_out : (k == 1 ? a.dbeta_out : a.dbias_out);
        if (out) *reinterpret_cast<float4*>(out + c) = t;
    }
}

// Teams: one workgroup per CU (fewer workgroups cannot draw the full HBM
// bandwidth) and no more, since each team writes one partial row of 3*h fp32
// that the finalize reads back.
int64_t bwd_teams(const spr_desc& d, const RowPlan& p) {
    const int64_t rows = d.s_local * d.b;
    const int64_t cap = 256 * (int64_t)p.rpw;       // one workgroup per CU
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
    if constexpr (WR) {
        switch (p.vpt) {
            SPR_BWD_CASE(1, 256) SPR_BWD_CASE(2, 256) SPR_BWD_CASE(3, 256) SPR_BWD_CASE(4, 256)
            default: return hipErrorInvalidValue;
        }
    } else {
        // must match kBwdCombos
        switch (p.vpt) {
            SPR_BWD_CASE(1, 1024) SPR_BWD_CASE(2, 768) SPR_BWD_CASE(3, 512)
            SPR_BWD_CASE(4, 512) SPR_BWD_CASE(5, 640) SPR_BWD_CASE(6, 512) SPR_BWD_CASE(8, 512)
            default: return hipErrorInvalidValue;
        }
    }
#undef SPR_BWD_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n3 = 3 * a.hidden;
    hipLaunchKernelGGL(sp_region_bwd_finalize_kernel, dim3((unsigned)((n3 + kFinCols - 1) / kFinCols)),
                       dim3(256), 0, s, a);
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
