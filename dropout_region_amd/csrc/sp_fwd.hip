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
// statistics written once; the row stays in registers from its load to its
// last store.  Two kernels: the row kernel (one team per row, parameters
// read per row from L2) and the stream kernel (a chip-filling grid walking
// rows with the next row's loads in flight, parameters held in registers).
// h is bit-exact: u, v and h are each a single fp32 operation rounded to
// nearest even (no contraction into FMA), then rounded to the I/O type.
#include <atomic>

#include "sp_device.h"
#include "sp_plan.h"

namespace spr {

// Pieces of one row's forward, shared by the two kernels below.  Thread
// `tid` of the row's team owns vectors vc[k] = k*tpr + tid (ok[k] false for
// the idle slots of a ragged row, which re-read the row's last vector and are
// masked afterwards).

// Dropout decisions, h = residual + dropout(x + bias) and its stores (h, and
// the mask when p > 0).  Element
// (row, c) is element e = (row_base + row)*h + c of the full tensor; its
// word is word e%4 of Philox block e/4.
template <typename IO, bool DROP, int VPT>
__device__ __forceinline__ void fwd_dropout_residual(const FwdArgs& a, int64_t row,
                                                      const int (&vc)[VPT], const bool (&ok)[VPT],
                                                      const uint4 (&xq)[VPT], const uint4 (&rq)[VPT],
                                                      const float (&bb)[VPT][Vec<IO>::N],
                                                      float (&hv)[VPT][Vec<IO>::N]) {
    constexpr int E = Vec<IO>::N;
    constexpr int MW = E / 4;                 // mask words per vector
    const int64_t rbase = row * a.hidden;
    if (!a.x) {                               // norm-only entry: h is the residual, bit for bit
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            Vec<IO> r;
            r.set(rq[k]);
#pragma unroll
            for (int j = 0; j < E; ++j) hv[k][j] = r.v[j];
            if (ok[k] && a.h_out)
                store_stream(static_cast<IO*>(a.h_out) + rbase + (int64_t)vc[k] * E, rq[k]);
        }
        return;
    }
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
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        uint4 hw;
        HVec<IO>::compute(xq[k], rq[k], bb[k], keep[k], DROP ? a.scale : 1.0f, hw, hv[k]);
        if (ok[k]) {
            const int64_t off = rbase + (int64_t)vc[k] * E;
            store_stream(static_cast<IO*>(a.h_out) + off, hw);
            if (DROP && a.mask_out) {         // no mask stored: the backward regenerates it
#pragma unroll
                for (int q = 0; q < MW; ++q)
                    __builtin_nontemporal_store(mask_word(&keep[k][4 * q]),
                                                reinterpret_cast<uint32_t*>(a.mask_out + off) + q);
            }
        }
    }
}

// The row's statistics over the team (one block reduction through `red`):
// LayerNorm merges each thread's (count, mean, M2) (Chan et al.), the means
// relative to a pivot (a value of the row, lane 0's first, per wave) so that
// a row whose mean dwarfs its spread keeps its variance; RMSNorm sums
// squares.  Returns mean (0 for RMSNorm), rstd, and for LayerNorm the pivot
// `piv` and the mean relative to it, `mrel` (mean = piv + mrel, rounded).
template <int NORM, int VPT, int E>
__device__ __forceinline__ void fwd_stats(const FwdArgs& a, const bool (&ok)[VPT],
                                          const float (&hv)[VPT][E], float* red, int nwaves,
                                          float& mean, float& rstd, float& piv, float& mrel) {
    float var;
    mean = 0.0f;
    piv = 0.0f;
    mrel = 0.0f;
    if (NORM == SPR_LAYERNORM) {
        // lane 0's first slot holds a value of the row (an idle slot re-reads
        // the row's last vector), uniform over the wave
        const float wpiv = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(hv[0][0])));
        float n = 0.0f, s = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            if (ok[k]) {
                n += (float)E;
#pragma unroll
                for (int j = 0; j < E; ++j) s += hv[k][j] - wpiv;
            }
        }
        const float m_loc = n > 0.0f ? s / n : 0.0f;       // relative to wpiv
        const float m_abs = wpiv + m_loc;
        float m2 = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            if (ok[k]) {
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const float d = hv[k][j] - m_abs;
                    m2 = fmaf(d, d, m2);
                }
            }
        }
        const MeanM2 st = block_mean_m2(MeanM2{n, m_loc, m2}, wpiv, red, nwaves, piv);
        mrel = st.mean;
        mean = piv + mrel;
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
    rstd = rsqrtf(var + a.eps);
}

// y = Norm(h) * gamma (+ beta) and the row's statistics.
template <typename IO, int NORM, int VPT>
__device__ __forceinline__ void fwd_store_y(const FwdArgs& a, int64_t row, int tid,
                                            const int (&vc)[VPT], const bool (&ok)[VPT],
                                            const float (&hv)[VPT][Vec<IO>::N],
                                            const float (&g)[VPT][Vec<IO>::N],
                                            const float (&bt)[VPT][Vec<IO>::N], float mean,
                                            float rstd, float piv, float mrel) {
    constexpr int E = Vec<IO>::N;
    const int64_t rbase = row * a.hidden;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (ok[k]) {
            Vec<IO> yv;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                // xhat = (h - mean) * rstd: the difference is exact for h
                // near the mean, so a row whose mean is many times its spread
                // (a constant row: rstd = 1/sqrt(eps)) keeps xhat accurate,
                // where h * rstd - mean * rstd would carry the rounding of
                // mean * rstd.  fp32 output also avoids the rounding of the
                // mean itself: (h - pivot) - mean relative to the pivot.
                float xh;
                if (NORM != SPR_LAYERNORM)
                    xh = hv[k][j] * rstd;
                else if (E == 4)                                  // fp32 I/O
                    xh = ((hv[k][j] - piv) - mrel) * rstd;
                else
                    xh = (hv[k][j] - mean) * rstd;
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

template <int VPT>
__device__ __forceinline__ void row_slots(int tid, int tpr, int nvec, bool exact, int (&vc)[VPT],
                                          bool (&ok)[VPT]) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        ok[k] = exact || vec < nvec;
        vc[k] = ok[k] ? vec : nvec - 1;
    }
}

template <typename IO, int VPT>
__device__ __forceinline__ void load_x_res(const FwdArgs& a, int64_t row, const int (&vc)[VPT],
                                           uint4 (&xq)[VPT], uint4 (&rq)[VPT]) {
    constexpr int E = Vec<IO>::N;
    const int64_t rbase = row * a.hidden;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        xq[k] = a.x ? load_stream(static_cast<const IO*>(a.x) + rbase + (int64_t)vc[k] * E)
                    : make_uint4(0u, 0u, 0u, 0u);
        rq[k] = load_stream(static_cast<const IO*>(a.residual) + rbase + (int64_t)vc[k] * E);
    }
}

// The reduce-scatter prologue: x = round_io(x_parts[0] + x_parts[1] + ...)
// over the row's vectors, fp32 adds in rank order, then one rounding to the
// I/O type.  Parts are loaded in groups of G, 8 vectors per thread in flight
// (a group slot past the last part re-reads part 0 and does not add it), so
// the prologue needs no more registers than the rest of the kernel.
template <typename IO, int VPT>
__device__ __forceinline__ void load_x_sum(const FwdArgs& a, int64_t row, const int (&vc)[VPT],
                                           uint4 (&xq)[VPT]) {
    using V = Vec<IO>;
    constexpr int E = V::N;
    const IO* base = static_cast<const IO*>(a.x) + row * a.hidden;
    float acc[VPT][E];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        V v;
        v.set(load_stream(base + (int64_t)vc[k] * E));
#pragma unroll
        for (int j = 0; j < E; ++j) acc[k][j] = v.v[j];
    }
    constexpr int G = VPT >= 8 ? 1 : 8 / VPT;
    for (int p0 = 1; p0 < a.nparts; p0 += G) {
        uint4 q[G][VPT];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int p = p0 + i < a.nparts ? p0 + i : 0;
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                q[i][k] = load_stream(base + (int64_t)p * a.part_stride + (int64_t)vc[k] * E);
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if (p0 + i < a.nparts) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    V v;
                    v.set(q[i][k]);
#pragma unroll
                    for (int j = 0; j < E; ++j) acc[k][j] += v.v[j];
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        V v;
#pragma unroll
        for (int j = 0; j < E; ++j) v.v[j] = acc[k][j];
        xq[k] = v.get();
    }
}

template <int VPT, int E>
__device__ __forceinline__ void load_bias(const FwdArgs& a, const int (&vc)[VPT],
                                          float (&bb)[VPT][E]) {
    if (a.bias) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) load_params<E>(a.bias + (int64_t)vc[k] * E, bb[k]);
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
            for (int j = 0; j < E; ++j) bb[k][j] = 0.0f;
    }
}

template <int NORM, int VPT, int E>
__device__ __forceinline__ void load_affine(const FwdArgs& a, const int (&vc)[VPT],
                                            float (&g)[VPT][E], float (&bt)[VPT][E]) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        load_params<E>(a.gamma + (int64_t)vc[k] * E, g[k]);
        if (NORM == SPR_LAYERNORM) load_params<E>(a.beta + (int64_t)vc[k] * E, bt[k]);
    }
}

// Row kernel: one team per row.  WAVE_ROWS: each wave owns one row (short
// rows, 4 rows per workgroup, no LDS); otherwise the whole workgroup owns
// one row.  EXACT: the row is exactly VPT vectors per thread.  With
// nparts > 1 it also runs the reduce-scatter prologue (x is the sum of
// nparts partial slabs).
//
// Every load is issued unconditionally, so a thread has all its x and
// residual vectors in flight at once; the dropout words, which need no
// data, are computed while they arrive.  bias, gamma and beta come from L2.
template <typename IO, int NORM, bool DROP, int VPT, bool WAVE_ROWS, int LB, bool EXACT>
__global__ void __launch_bounds__(LB) sp_region_fwd_kernel(FwdArgs a) {
    constexpr int E = Vec<IO>::N;
    __shared__ float red[64];

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

    int vc[VPT];
    bool ok[VPT];
    row_slots<VPT>(tid, tpr, a.nvec, EXACT, vc, ok);
    uint4 xq[VPT], rq[VPT];
    if (a.nparts > 1) {                  // uniform: the reduce-scatter prologue
        const IO* rr = static_cast<const IO*>(a.residual) + row * a.hidden;
#pragma unroll
        for (int k = 0; k < VPT; ++k) rq[k] = load_stream(rr + (int64_t)vc[k] * E);
        load_x_sum<IO, VPT>(a, row, vc, xq);
    } else {
        load_x_res<IO, VPT>(a, row, vc, xq, rq);
    }
    float bb[VPT][E];
    load_bias<VPT, E>(a, vc, bb);

    float hv[VPT][E];
    fwd_dropout_residual<IO, DROP, VPT>(a, row, vc, ok, xq, rq, bb, hv);
    if (!a.gamma) return;                // norm-free exit: h and the mask only (uniform)

    float g[VPT][E], bt[VPT][E];
    load_affine<NORM, VPT, E>(a, vc, g, bt);
    float mean, rstd, piv, mrel;
    fwd_stats<NORM, VPT, E>(a, ok, hv, red, nwaves, mean, rstd, piv, mrel);
    fwd_store_y<IO, NORM, VPT>(a, row, tid, vc, ok, hv, g, bt, mean, rstd, piv, mrel);
}

// Stream kernel: a grid of G workgroups, about as many as fit on the chip at
// once; workgroup b owns rows b, b + G, b + 2G, ...  bias, gamma and beta are
// the same columns for every row, so they are loaded once and held; the next
// row's x and residual are loaded before the current row is computed, so its
// loads are in flight during the current row's arithmetic, reduction and
// stores.  Two register sets alternate (A computes while B loads, then B
// computes while A loads).  The LDS reduction slots alternate too, so a
// row's reduction never overwrites a slot that a slower wave may still be
// reading for the previous row.
template <typename IO, int NORM, bool DROP, int VPT, int LB, bool EXACT>
__global__ void __launch_bounds__(LB) sp_region_fwd_stream_kernel(FwdArgs a) {
    constexpr int E = Vec<IO>::N;
    __shared__ float red[2][64];
    const int tid = threadIdx.x, tpr = blockDim.x, nwaves = blockDim.x >> 6;
    const int64_t step = gridDim.x;

    int vc[VPT];
    bool ok[VPT];
    row_slots<VPT>(tid, tpr, a.nvec, EXACT, vc, ok);

    int64_t row = blockIdx.x;          // uniform over the workgroup
    if (row >= a.rows) return;
    uint4 xa[VPT], ra[VPT], xb[VPT], rb[VPT];
    load_x_res<IO, VPT>(a, row, vc, xa, ra);
    float bb[VPT][E], g[VPT][E], bt[VPT][E];
    load_bias<VPT, E>(a, vc, bb);
    if (a.gamma) load_affine<NORM, VPT, E>(a, vc, g, bt);

    auto one_row = [&](int64_t r, const uint4 (&xq)[VPT], const uint4 (&rq)[VPT], float* slot) {
        float hv[VPT][E];
        fwd_dropout_residual<IO, DROP, VPT>(a, r, vc, ok, xq, rq, bb, hv);
        if (!a.gamma) return;            // norm-free exit (uniform)
        float mean, rstd, piv, mrel;
        fwd_stats<NORM, VPT, E>(a, ok, hv, slot, nwaves, mean, rstd, piv, mrel);
        fwd_store_y<IO, NORM, VPT>(a, r, tid, vc, ok, hv, g, bt, mean, rstd, piv, mrel);
    };
    for (;;) {
        if (row + step < a.rows) load_x_res<IO, VPT>(a, row + step, vc, xb, rb);
        one_row(row, xa, ra, red[0]);
        row += step;
        if (row >= a.rows) break;
        if (row + step < a.rows) load_x_res<IO, VPT>(a, row + step, vc, xa, ra);
        one_row(row, xb, rb, red[1]);
        row += step;
        if (row >= a.rows) break;
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

// ---------------------------------------------------------------- stream kernel dispatch
// Workgroups of a stream kernel: per CU, enough for at least 8 waves (as
// many as fit, if fewer), then trimmed so that every workgroup gets the same
// number of rows (or one fewer).  `occ` is how many of its workgroups fit on
// a CU.
static int64_t stream_grid(int occ, int block, int64_t rows, int cus) {
    const int waves = (block + 63) / 64;
    int per_cu = (8 + waves - 1) / waves;
    if (per_cu > occ) per_cu = occ;
    const int64_t cap = (int64_t)per_cu * cus;
    const int64_t per_wg = (rows + cap - 1) / cap;
    return (rows + per_wg - 1) / per_wg;
}

template <typename IO, int NORM, bool DROP, int V, bool EXACT>
static hipError_t fwd_stream_launch(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    constexpr int LB = stream_bound(Vec<IO>::N, V);
    auto kernel = sp_region_fwd_stream_kernel<IO, NORM, DROP, V, LB, EXACT>;
    // Workgroups of this instantiation that fit on a CU, kept with the block
    // size they were queried for; a launch with another block size queries
    // again.
    static std::atomic<int64_t> fit{0};     // (block << 32) | occupancy
    const int64_t f = fit.load(std::memory_order_relaxed);
    int occ = (f >> 32) == p.block ? (int)(f & 0xffffffff) : 0;
    if (occ == 0) {
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, p.block, 0);
        if (e != hipSuccess) return e;
        if (occ < 1) occ = 1;
        fit.store(((int64_t)p.block << 32) | occ, std::memory_order_relaxed);
    }
    const int64_t grid = stream_grid(occ, p.block, a.rows, device_cu_count());
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3((unsigned)p.block), 0, s, a);
    return hipGetLastError();
}

template <typename IO, int NORM, bool DROP, bool EXACT>
static hipError_t fwd_stream_by_vpt(const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    if constexpr (Vec<IO>::N == 8) {
        switch (p.vpt) {
            case 1: return fwd_stream_launch<IO, NORM, DROP, 1, EXACT>(p, a, s);
            case 2: return fwd_stream_launch<IO, NORM, DROP, 2, EXACT>(p, a, s);
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.vpt) {
            case 1: return fwd_stream_launch<IO, NORM, DROP, 1, EXACT>(p, a, s);
            case 2: return fwd_stream_launch<IO, NORM, DROP, 2, EXACT>(p, a, s);
            case 3: return fwd_stream_launch<IO, NORM, DROP, 3, EXACT>(p, a, s);
            case 4: return fwd_stream_launch<IO, NORM, DROP, 4, EXACT>(p, a, s);
            default: return hipErrorInvalidValue;
        }
    }
}

template <typename IO, int NORM>
static hipError_t fwd_stream_by_mode(const spr_desc& d, const RowPlan& p, const FwdArgs& a,
                                     hipStream_t s) {
    const bool exact = p.nvec == p.vpt * p.tpr;
    if (d.p > 0.0f)
        return exact ? fwd_stream_by_vpt<IO, NORM, true, true>(p, a, s)
                     : fwd_stream_by_vpt<IO, NORM, true, false>(p, a, s);
    return exact ? fwd_stream_by_vpt<IO, NORM, false, true>(p, a, s)
                 : fwd_stream_by_vpt<IO, NORM, false, false>(p, a, s);
}

template <typename IO>
static hipError_t fwd_stream_by_norm(const spr_desc& d, const RowPlan& p, const FwdArgs& a,
                                     hipStream_t s) {
    return d.norm == SPR_LAYERNORM ? fwd_stream_by_mode<IO, SPR_LAYERNORM>(d, p, a, s)
                                   : fwd_stream_by_mode<IO, SPR_RMSNORM>(d, p, a, s);
}

// The row kernel by default.  The stream kernel (where its plan exists: at
// most 16 elements per thread, so bias, gamma and beta fit in registers next
// to two row buffers) runs when desc.fwd_kernel asks for it; measured on
// MI355X it is no faster anywhere the row kernel takes its preferred split
// (long-sequence shard [4096, 1, 8192]: row kernel 59.2 us against 60.7 at
// p = 0.1, 51.1 against 53.8 at p = 0).
hipError_t launch_fwd(const spr_desc& d, const RowPlan& p, const FwdArgs& a, hipStream_t s) {
    RowPlan sp;
    bool stream = d.fwd_kernel == SPR_FWD_STREAM && make_stream_plan(d.io, d.h, &sp);
    if (a.nparts > 1) stream = false;    // the prologue is in the row kernel only
    if (stream)
        return d.io == SPR_BF16 ? fwd_stream_by_norm<__bf16>(d, sp, a, s)
                                : fwd_stream_by_norm<float>(d, sp, a, s);
    return d.io == SPR_BF16 ? fwd_by_norm<__bf16>(d, p, a, s) : fwd_by_norm<float>(d, p, a, s);
}

}  // namespace spr
