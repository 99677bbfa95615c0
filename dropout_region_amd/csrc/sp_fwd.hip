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
// LDS); otherwise the whole workgroup owns one row.
template <typename IO, int NORM, bool DROP, int VPT, bool WAVE_ROWS, int LB>
__global__ void __launch_bounds__(LB) sp_region_fwd_kernel(FwdArgs a) {
    using V = Vec<IO>;
    constexpr int E = V::N;
    __shared__ float red[2][16];

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

    const IO* xr = static_cast<const IO*>(a.x) + row * a.hidden;
    const IO* rr = static_cast<const IO*>(a.residual) + row * a.hidden;

    V xv[VPT], rv[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        if (vec < a.nvec) {
            xv[k].load(xr + (int64_t)vec * E);
            rv[k].load(rr + (int64_t)vec * E);
        }
    }

    // Dropout decisions: element (row, c) is element e = (row_base+row)*h + c
    // of the full tensor; its word is word e%4 of Philox block e/4.
    uint32_t kb[VPT];
    if (DROP) {
        const uint64_t e_row = (a.row_base + (uint64_t)row) * (uint64_t)a.hidden;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int vec = k * tpr + tid;
            const uint64_t blk = (e_row + (uint64_t)vec * E) >> 2;
            uint32_t bits = keep4(blk, a.off_lo, a.off_hi, a.key_lo, a.key_hi, a.thr);
            if (E == 8) bits |= keep4(blk + 1, a.off_lo, a.off_hi, a.key_lo, a.key_hi, a.thr) << 4;
            kb[k] = bits;
        }
    }

    float hv[VPT][E];
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        if (vec < a.nvec) {
            float bb[E];
            if (a.bias) {
                load_params<E>(a.bias + (int64_t)vec * E, bb);
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) bb[j] = 0.0f;
            }
            V hvec;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                // p == 0: every element is kept and scale is exactly 1
                const bool keep = DROP ? ((kb[k] >> j) & 1u) != 0 : true;
                const float hr = V::round_io(
                    residual_dropout(xv[k].v[j], bb[j], rv[k].v[j], keep, DROP ? a.scale : 1.0f));
                hv[k][j] = hr;
                hvec.v[j] = hr;
                sum += hr;
            }
            const int64_t off = row * a.hidden + (int64_t)vec * E;
            hvec.store(static_cast<IO*>(a.h_out) + off);
            if (DROP) MaskBytes<E>::store(a.mask_out + off, kb[k]);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) hv[k][j] = 0.0f;
        }
    }

    float mean = 0.0f;
    if (NORM == SPR_LAYERNORM) mean = block_sum(sum, red[0], nwaves) * a.inv_h;
    float sq = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        if (vec < a.nvec) {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float d = hv[k][j] - mean;
                sq += d * d;
            }
        }
    }
    sq = block_sum(sq, red[1], nwaves);
    const float rstd = rsqrtf(sq * a.inv_h + a.eps);

#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        if (vec < a.nvec) {
            float g[E], b[E];
            load_params<E>(a.gamma + (int64_t)vec * E, g);
            if (NORM == SPR_LAYERNORM) load_params<E>(a.beta + (int64_t)vec * E, b);
            V yv;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float xh = (hv[k][j] - mean) * rstd;
                yv.v[j] = (NORM == SPR_LAYERNORM) ? xh * g[j] + b[j] : xh * g[j];
            }
            yv.store(static_cast<IO*>(a.y_out) + row * a.hidden + (int64_t)vec * E);
        }
    }
    if (tid == 0) {
        if (NORM == SPR_LAYERNORM) a.mean_out[row] = mean;
        a.rstd_out[row] = rstd;
    }
}

template <typename IO, int NORM, bool DROP, bool WR>
static hipError_t fwd_by_vpt(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    const int64_t grid = WR ? (a.rows + p.rpw - 1) / p.rpw : a.rows;
    const dim3 g((unsigned)grid), b((unsigned)p.block);
#define SPR_FWD_CASE(V, L)                                                                    \
    case V:                                                                                   \
        hipLaunchKernelGGL((sp_region_fwd_kernel<IO, NORM, DROP, V, WR, L>), g, b, 0, s, a);  \
        break;
    if (WR) {
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
    return p.rpw > 1 ? fwd_by_vpt<IO, NORM, DROP, true>(p, a, s)
                     : fwd_by_vpt<IO, NORM, DROP, false>(p, a, s);
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
