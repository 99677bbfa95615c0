// sp_fwd.hip -- forward of the sequence-parallel region on gfx950.
//
// Per token row (the band is per token: "Sequence parallel math", section
// "The move: split the LayerNorm/dropout band along the sequence"; "SP:
// Partition Activations Alongside TP", section "Normalize and add residuals
// by token"):
//   u = x + bias, keep = Philox(e) >= thr, h = round_io(residual + (keep ? u*scale : 0))
//   mean/rstd of the rounded h, y = (h - mean) * rstd * gamma + beta (RMSNorm:
//   y = h * rstd * gamma).
// One pass over HBM: x and residual are read once, h, mask, y and the two
// statistics written once; the row stays in registers between the two
// reductions (mean, then the centred sum of squares).  Bias/gamma/beta are
// re-read per row and come from L2.  h is bit-exact: u, v and h are each a
// single fp32 operation rounded to nearest even (no contraction into FMA),
// then rounded to the I/O type.
#include "sp_device.h"
#include "sp_plan.h"

namespace spr {

// WAVE_ROWS: each wave owns one row (short rows, 4 rows per workgroup, no
// LDS); otherwise the whole workgroup owns one row.  EXACT: the row is
// exactly VPT vectors per thread, so no slot is idle.
//
// Every load is issued unconditionally (a ragged row's idle slots re-read its
// last vector and are masked afterwards), so a thread has all its x and
// residual vectors in flight at once; the dropout words, which need no
// data, are computed while they arrive.  Statistics: each thread reduces
// its own values to (count, mean, M2), then one Chan merge over the team.
template <typename IO, int NORM, bool DROP, int VPT, bool WAVE_ROWS, int LB, bool EXACT>
__global__ void __launch_bounds__(LB) sp_region_fwd_kernel(FwdArgs a) {
    constexpr int E = Vec<IO>::N;
    constexpr int MW = E / 4;                 // mask words per vector
    __shared__ float red[48];

    int tid, tpr, nwaves;
    int64_t row;
    if (WAVE_ROWS) {
        tid = threadIdx.x & 63;
        tpr = 64;
        nwaves = 1;
        row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    } else {
        tid = threadIdx.x;
        tpr = blockDim.x;
        nwaves = blockDim.x >> 6;
        row = blockIdx.x;
    }
    // Uniform per wave (WAVE_ROWS) or per workgroup: no barrier is skipped
    // by part of a team.
    if (row >= a.rows) return;

    const int64_t rbase = row * a.hidden;
    const IO* xr = static_cast<const IO*>(a.x) + rbase;
    const IO* rr = static_cast<const IO*>(a.residual) + rbase;

    int vc[VPT];
    bool ok[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        ok[k] = EXACT || vec < a.nvec;
        vc[k] = ok[k] ? vec : a.nvec - 1;
    }

    uint4 xq[VPT], rq[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        xq[k] = load_stream(xr + (int64_t)vc[k] * E);
        rq[k] = load_stream(rr + (int64_t)vc[k] * E);
    }
    float bb[VPT][E];
    if (a.bias) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) load_params<E>(a.bias + (int64_t)vc[k] * E, bb[k]);
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
            for (int j = 0; j < E; ++j) bb[k][j] = 0.0f;
    }

    // Dropout decisions: element (row, c) is element e = (row_base+row)*h + c
    // of the full tensor; its word is word e%4 of Philox block e/4.
    bool keep[VPT][E];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (DROP) {
            const uint64_t e0 = (a.row_base + (uint64_t)row) * (uint64_t)a.hidden +
                                (uint64_t)vc[k] * E;
#pragma unroll
            for (int q = 0; q < MW; ++q)
                keep4((e0 >> 2) + q, a.off_lo, a.off_hi, a.key_lo, a.key_hi, a.thr, &keep[k][4 * q]);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) keep[k][j] = true;   // p == 0: scale is exactly 1
        }
    }

    float hv[VPT][E];
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        uint4 hw;
        HVec<IO>::compute(xq[k], rq[k], bb[k], keep[k], DROP ? a.scale : 1.0f, hw, hv[k]);
        if (ok[k]) {
#pragma unroll
            for (int j = 0; j < E; ++j) sum += hv[k][j];
            const int64_t off = rbase + (int64_t)vc[k] * E;
            store_stream(static_cast<IO*>(a.h_out) + off, hw);
            if (DROP) {
#pragma unroll
                for (int q = 0; q < MW; ++q)
                    __builtin_nontemporal_store(mask_word(&keep[k][4 * q]),
                                                reinterpret_cast<uint32_t*>(a.mask_out + off) + q);
            }
        }
    }

    float g[VPT][E], bt[VPT][E];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        load_params<E>(a.gamma + (int64_t)vc[k] * E, g[k]);
        if (NORM == SPR_LAYERNORM) load_params<E>(a.beta + (int64_t)vc[k] * E, bt[k]);
    }

    float mean = 0.0f, var;
    if (NORM == SPR_LAYERNORM) {
        float n = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) n += ok[k] ? (float)E : 0.0f;
        const float m_loc = n > 0.0f ? sum / n : 0.0f;
        float m2 = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            if (ok[k]) {
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const float d = hv[k][j] - m_loc;
                    m2 = fmaf(d, d, m2);
                }
            }
        }
        const MeanM2 st = block_mean_m2(MeanM2{n, m_loc, m2}, red, nwaves);
        mean = st.mean;
        var = st.m2 * a.inv_h;
    } else {
        float sq = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            if (ok[k]) {
#pragma unroll
                for (int j = 0; j < E; ++j) sq = fmaf(hv[k][j], hv[k][j], sq);
            }
        }
        var = block_sum(sq, red, nwaves) * a.inv_h;     // mean square
    }
    const float rstd = rsqrtf(var + a.eps);
    const float shift = -mean * rstd;                   // xhat = h * rstd + shift

#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (ok[k]) {
            Vec<IO> yv;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float xh = fmaf(hv[k][j], rstd, shift);
                yv.v[j] = (NORM == SPR_LAYERNORM) ? fmaf(xh, g[k][j], bt[k][j]) : xh * g[k][j];
            }
            yv.store(static_cast<IO*>(a.y_out) + rbase + (int64_t)vc[k] * E);
        }
    }
    if (tid == 0) {
        if (NORM == SPR_LAYERNORM) a.mean_out[row] = mean;
        a.rstd_out[row] = rstd;
    }
}

template <typename IO, int NORM, bool DROP, bool WR, bool EXACT>
static hipError_t fwd_by_vpt(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    const int64_t grid = WR ? (a.rows + p.rpw - 1) / p.rpw : a.rows;
    const dim3 g((unsigned)grid), b((unsigned)p.block);
#define SPR_FWD_CASE(V, L)                                                                    \
    case V:                                                                                   \
        hipLaunchKernelGGL((sp_region_fwd_kernel<IO, NORM, DROP, V, WR, L, EXACT>), g, b, 0, s, a); \
        break;
    if constexpr (WR) {
        switch (p.vpt) {
            SPR_FWD_CASE(1, 256) SPR_FWD_CASE(2, 256) SPR_FWD_CASE(3, 256) SPR_FWD_CASE(4, 256)
            default: return hipErrorInvalidValue;
        }
    } else {
        // must match kWgCombos
        switch (p.vpt) {
            SPR_FWD_CASE(1, 1024) SPR_FWD_CASE(2, 1024) SPR_FWD_CASE(3, 1024)
            SPR_FWD_CASE(4, 1024) SPR_FWD_CASE(5, 768) SPR_FWD_CASE(6, 768) SPR_FWD_CASE(8, 512)
            default: return hipErrorInvalidValue;
        }
    }
#undef SPR_FWD_CASE
    return hipGetLastError();
}

template <typename IO, int NORM, bool DROP>
static hipError_t fwd_by_mode(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    const bool exact = p.nvec == p.vpt * p.tpr;
    if (p.rpw > 1)
        return exact ? fwd_by_vpt<IO, NORM, DROP, true, true>(p, a, s)
                     : fwd_by_vpt<IO, NORM, DROP, true, false>(p, a, s);
    return exact ? fwd_by_vpt<IO, NORM, DROP, false, true>(p, a, s)
                 : fwd_by_vpt<IO, NORM, DROP, false, false>(p, a, s);
}

template <typename IO, int NORM>
static hipError_t fwd_by_drop(const spr_desc& d, const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    return d.p > 0.0f ? fwd_by_mode<IO, NORM, true>(p, a, s) : fwd_by_mode<IO, NORM, false>(p, a, s);
}

template <typename IO>
static hipError_t fwd_by_norm(const spr_desc& d, const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    return d.norm == SPR_LAYERNORM ? fwd_by_drop<IO, SPR_LAYERNORM>(d, p, a, s)
                                   : fwd_by_drop<IO, SPR_RMSNORM>(d, p, a, s);
}

hipError_t launch_fwd(const spr_desc& d, const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    return d.io == SPR_BF16 ? fwd_by_norm<__bf16>(d, p, a, s) : fwd_by_norm<float>(d, p, a, s);
}

}  // namespace spr
