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

// Keep decision of element j of a vector from its mask words (one byte per
// element; any nonzero byte keeps).
template <int MW>
__device__ __forceinline__ bool mask_keeps(const uint32_t (&w)[MW], int j) {
    return ((w[j >> 2] >> (8 * (j & 3))) & 0xffu) != 0u;
}

// EXACT: every vector slot of the team holds a vector of the row (no idle
// slot to mask out of the sums).
template <typename IO, int NORM, int DROP, int VPT, bool WAVE_ROWS, int LB, bool EXACT>
__global__ void __launch_bounds__(LB) sp_region_bwd_rows_kernel(BwdArgs a) {
    // Rows in flight per thread (each costs the row's registers again).
    constexpr int DEPTH = bwd_depth(VPT, LB, WAVE_ROWS, NORM == SPR_LAYERNORM);
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
        ok[k] = EXACT || vec < a.nvec;
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
            if (DROP == kDropMask) {
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

    // One row: the two row sums (one team reduction through `slot`), then
    // dx/dresidual and the column partials.  With d = h - mean (RMSNorm:
    // d = h), xhat = d * rstd and g = dy * gamma,
    //   dh = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat))
    //      = rstd * g - c1 - c2 * d,   c1 = rstd * mean_c(g),
    //                                  c2 = rstd^3 * mean_c(g * d)
    // (RMSNorm: c1 = 0), two FMAs per element after the row constants.
    auto process = [&](int64_t row, const RowIn<VPT, MW>& cur, float* slot) {
        // Regenerated dropout: the row's keep bits.
        uint32_t kbits[VPT];
        if (DROP == kDropRegen) {
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                kbits[k] = keep_bits<E>((a.row_base + (uint64_t)row) * (uint64_t)a.hidden +
                                            (uint64_t)vc[k] * E,
                                        a.off_lo, a.off_hi, a.key_lo, a.key_hi, a.thr);
        }

        const float rs = cur.rs;
        float d[VPT][E], dyf[VPT][E];
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            V hv, dv;
            hv.set(cur.h[k]);
            dv.set(cur.dy[k]);
#pragma unroll
            for (int j = 0; j < E; ++j) {
                d[k][j] = (NORM == SPR_LAYERNORM) ? hv.v[j] - cur.mu : hv.v[j];
                dyf[k][j] = dv.v[j];
                const float g = dv.v[j] * gam[k][j];
                if (ok[k]) {
                    s1 += g;
                    s2 = fmaf(g, d[k][j], s2);
                }
            }
        }
        block_sum2(s1, s2, slot, nwaves);
        const float c1 = (NORM == SPR_LAYERNORM) ? rs * (s1 * a.inv_h) : 0.0f;
        const float c2 = rs * (rs * (rs * (s2 * a.inv_h)));   // 0 when s2 is, whatever rs

        const int64_t rbase = row * a.hidden;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            V dho, dres, dx;
            if (a.dh_out) dho.set(cur.dho[k]);
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float g = dyf[k][j] * gam[k][j];
                float dh = fmaf(rs, g, fmaf(-c2, d[k][j], -c1));
                if (a.dh_out) dh += dho.v[j];
                bool keep = true;
                if (DROP == kDropMask) keep = mask_keeps<MW>(cur.mask[k], j);
                else if (DROP == kDropRegen) keep = ((kbits[k] >> j) & 1u) != 0u;
                const float dxu = DROP != kDropNone ? (keep ? dh * a.scale : 0.0f) : dh;
                dres.v[j] = dh;
                dx.v[j] = dxu;
                if (ok[k]) {
                    acc_g[k][j] = fmaf(dyf[k][j], d[k][j] * rs, acc_g[k][j]);
                    acc_b[k][j] += dyf[k][j];
                    acc_x[k][j] += dxu;
                }
            }
            if (ok[k]) {
                const int64_t off = rbase + (int64_t)vc[k] * E;
                dres.store(static_cast<IO*>(a.dres_out) + off);
                if (a.dx_out) dx.store(static_cast<IO*>(a.dx_out) + off);
            }
        }
    };

    // Rows team, team + teams, ...: the trip count is uniform over the team
    // (the workgroup, when the workgroup is the team), so every thread meets
    // every barrier.  Consecutive rows alternate the two reduction slots.
    // Narrow rows keep DEPTH rows in flight: a ring of DEPTH row buffers,
    // each refilled with the row DEPTH steps ahead as soon as its row is
    // done, so DEPTH - 1 rows are loading while one is computed.
    int slot = 0;
    if constexpr (DEPTH > 1) {
        RowIn<VPT, MW> buf[DEPTH];
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            const int64_t r = team + i * a.teams;
            if (r < a.rows) load_row(r, buf[i]);
        }
        int64_t row = team;
        bool more = row < a.rows;
        while (more) {
#pragma unroll
            for (int i = 0; i < DEPTH; ++i) {
                if (more) {
                    process(row, buf[i], red[slot]);
                    slot ^= 1;
                    const int64_t ahead = row + DEPTH * a.teams;
                    if (ahead < a.rows) load_row(ahead, buf[i]);
                    row += a.teams;
                    more = row < a.rows;
                }
            }
        }
    } else {
        RowIn<VPT, MW> cur;
        for (int64_t row = team; row < a.rows; row += a.teams) {
            load_row(row, cur);
            process(row, cur, red[slot]);
            slot ^= 1;
        }
    }

    float* part = a.partials + team * a.slots * a.hidden;
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
    const int64_t n3 = (int64_t)a.slots * a.hidden;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j < n3) {
        // Group q's teams q, q+16, ... in order, four loads in flight at a
        // time: stream i of the four takes every fourth of them, and the four
        // streams are added pairwise at the end -- a fixed order.
        const float* p = a.partials + j;
        float4 s4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int t = q; t < a.teams; t += 4 * kFinGroups) {
            float4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ti = t + i * kFinGroups;
                v[i] = ti < a.teams ? *reinterpret_cast<const float4*>(p + (int64_t)ti * n3)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s4[i].x += v[i].x; s4[i].y += v[i].y; s4[i].z += v[i].z; s4[i].w += v[i].w;
            }
        }
        s.x = (s4[0].x + s4[1].x) + (s4[2].x + s4[3].x);
        s.y = (s4[0].y + s4[1].y) + (s4[2].y + s4[3].y);
        s.z = (s4[0].z + s4[1].z) + (s4[2].z + s4[3].z);
        s.w = (s4[0].w + s4[1].w) + (s4[2].w + s4[3].w);
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
        float* out = a.slots == 1 ? a.dbias_out
                                  : (k == 0 ? a.dgamma_out : (k == 1 ? a.dbeta_out : a.dbias_out));
        if (out) *reinterpret_cast<float4*>(out + c) = t;
    }
}

// ---------------------------------------------------------------- split path
// Pass 1 (rowsum): one team per row, like the forward; reads dy and h and
// writes the row's two sums sum_c g and sum_c g*xhat (g = dy*gamma) to
// rowsum[row].  Pass 2 (main): tiles of tile_rows rows x one wave's 64
// vectors (512 bf16 / 256 fp32 columns); the workgroup's 4 waves take rows
// w, w + 4, ... and prefetch the next group of U rows while computing the
// current one; dx/dresidual are written and the dgamma/dbeta/dbias column
// partials of the tile's rows are added across the waves in wave order.
constexpr int kSplitWaves = 4, kSplitUnroll = 4;

template <typename IO, int NORM, int VPT, bool WAVE_ROWS, int LB, bool EXACT>
__global__ void __launch_bounds__(LB) sp_region_bwd_rowsum_kernel(BwdArgs a) {
    constexpr int E = Vec<IO>::N;
    __shared__ float red[32];
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
    if (row >= a.rows) return;               // uniform per wave / workgroup

    int vc[VPT];
    bool ok[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int vec = k * tpr + tid;
        ok[k] = EXACT || vec < a.nvec;
        vc[k] = ok[k] ? vec : a.nvec - 1;
    }
    const int64_t rbase = row * a.hidden;
    uint4 hq[VPT], dq[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        hq[k] = load_stream(static_cast<const IO*>(a.h) + rbase + (int64_t)vc[k] * E);
        dq[k] = load_stream(static_cast<const IO*>(a.dy) + rbase + (int64_t)vc[k] * E);
    }
    float gam[VPT][E];
#pragma unroll
    for (int k = 0; k < VPT; ++k) load_params<E>(a.gamma + (int64_t)vc[k] * E, gam[k]);
    const float mu = (NORM == SPR_LAYERNORM) ? a.mean[row] : 0.0f;
    const float rs = a.rstd[row];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        Vec<IO> hv, dv;
        hv.set(hq[k]);
        dv.set(dq[k]);
        if (ok[k]) {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float g = dv.v[j] * gam[k][j];
                s1 += g;
                s2 = fmaf(g, (hv.v[j] - mu) * rs, s2);
            }
        }
    }
    block_sum2(s1, s2, red, nwaves);
    if (tid == 0) *reinterpret_cast<float2*>(a.rowpart + row * 2) = make_float2(s1, s2);
}

// Adds the 4 waves' column partials in wave order and writes them as
// partial row `slot` of row block blockIdx.y: colpart[(rb*slots + slot)*h + c].
template <int E>
__device__ __forceinline__ void split_store_colpart(const BwdArgs& a, float (*sh)[64][E],
                                                    const float (&acc)[E], int slot, int vec,
                                                    bool ok) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < E; ++j) sh[wave][lane][j] = acc[j];
    __syncthreads();
    if (wave == 0 && ok) {
        float t[E];
#pragma unroll
        for (int j = 0; j < E; ++j) t[j] = sh[0][lane][j];
        for (int w = 1; w < kSplitWaves; ++w)
#pragma unroll
            for (int j = 0; j < E; ++j) t[j] += sh[w][lane][j];
        float* out = a.partials + ((int64_t)blockIdx.y * a.slots + slot) * a.hidden +
                     (int64_t)vec * E;
#pragma unroll
        for (int j = 0; j < E; j += 4)
            *reinterpret_cast<float4*>(out + j) = make_float4(t[j], t[j + 1], t[j + 2], t[j + 3]);
    }
    __syncthreads();
}

// The saved tensors of one group of U rows of a pass-2 tile (one vector each).
template <int U, int MW>
struct TileIn {
    uint4 h[U], dy[U], dho[U];
    uint32_t mask[U][MW];
    float mu[U], rs[U];
    float2 rsum[U];
};

template <typename IO, int NORM, int DROP>
__global__ void __launch_bounds__(256) sp_region_bwd_main_kernel(BwdArgs a) {
    using V = Vec<IO>;
    constexpr int E = V::N, U = kSplitUnroll, MW = E / 4;
    __shared__ float sh[kSplitWaves][64][E];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int vec = blockIdx.x * 64 + lane;
    const bool ok = vec < a.nvec;
    const int vcl = ok ? vec : a.nvec - 1;
    float gam[E], acc_g[E], acc_b[E], acc_x[E];
    load_params<E>(a.gamma + (int64_t)vcl * E, gam);
#pragma unroll
    for (int j = 0; j < E; ++j) acc_g[j] = acc_b[j] = acc_x[j] = 0.0f;

    const int64_t r0 = (int64_t)blockIdx.y * a.tile_rows;
    const int64_t r1 = r0 + a.tile_rows < a.rows ? r0 + a.tile_rows : a.rows;
    constexpr int64_t step = kSplitWaves * U;

    auto load_group = [&](int64_t base, TileIn<U, MW>& in) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + kSplitWaves * u;
            const int64_t rc = row < r1 ? row : r1 - 1;          // clamp: always a valid row
            const int64_t off = rc * a.hidden + (int64_t)vcl * E;
            in.h[u] = load_stream(static_cast<const IO*>(a.h) + off);
            in.dy[u] = load_stream(static_cast<const IO*>(a.dy) + off);
            if (DROP == kDropMask) {
#pragma unroll
                for (int w = 0; w < MW; ++w)
                    in.mask[u][w] = __builtin_nontemporal_load(
                        reinterpret_cast<const uint32_t*>(a.mask + off) + w);
            }
            if (a.dh_out) in.dho[u] = load_stream(static_cast<const IO*>(a.dh_out) + off);
            in.mu[u] = (NORM == SPR_LAYERNORM) ? a.mean[rc] : 0.0f;
            in.rs[u] = a.rstd[rc];
            in.rsum[u] = *reinterpret_cast<const float2*>(a.rowpart + rc * 2);
        }
    };

    auto process_group = [&](int64_t base, const TileIn<U, MW>& cur) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + kSplitWaves * u;
            const bool rok = row < r1;                       // wave-uniform
            const float mg = cur.rsum[u].x * a.inv_h, mgx = cur.rsum[u].y * a.inv_h;
            const float mu = cur.mu[u], rs = cur.rs[u];
            V hv, dv, dho, dres, dx;
            hv.set(cur.h[u]);
            dv.set(cur.dy[u]);
            if (a.dh_out) dho.set(cur.dho[u]);
            uint32_t kb = 0xffu;
            if (DROP == kDropMask) {
                kb = MaskBytes<4>::from_word(cur.mask[u][0]);
                if (MW == 2) kb |= MaskBytes<4>::from_word(cur.mask[u][MW - 1]) << 4;
            } else if (DROP == kDropRegen) {
                kb = keep_bits<E>((a.row_base + (uint64_t)row) * (uint64_t)a.hidden +
                                      (uint64_t)vcl * E,
                                  a.off_lo, a.off_hi, a.key_lo, a.key_hi, a.thr);
            }
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float xh = (hv.v[j] - mu) * rs;
                const float g = dv.v[j] * gam[j];
                float dh = (NORM == SPR_LAYERNORM) ? rs * (g - mg - xh * mgx)
                                                   : rs * (g - xh * mgx);
                if (a.dh_out) dh += dho.v[j];
                const float dxu =
                    DROP != kDropNone ? (((kb >> j) & 1u) ? dh * a.scale : 0.0f) : dh;
                dres.v[j] = dh;
                dx.v[j] = dxu;
                if (ok && rok) {
                    acc_g[j] = fmaf(dv.v[j], xh, acc_g[j]);
                    acc_b[j] += dv.v[j];
                    acc_x[j] += dxu;
                }
            }
            if (ok && rok) {
                const int64_t off = row * a.hidden + (int64_t)vec * E;
                dres.store(static_cast<IO*>(a.dres_out) + off);
                if (a.dx_out) dx.store(static_cast<IO*>(a.dx_out) + off);
            }
        }
    };

    // Trip counts differ between waves (ragged tiles) but nothing in the loop
    // synchronises the workgroup.
    TileIn<U, MW> cur, nxt;
    int64_t base = r0 + wave;
    if (base < r1) load_group(base, cur);
    for (; base < r1; base += step) {
        if (base + step < r1) load_group(base + step, nxt);
        process_group(base, cur);
        cur = nxt;
    }
    split_store_colpart<E>(a, sh, acc_g, 0, vec, ok);
    split_store_colpart<E>(a, sh, acc_b, 1, vec, ok);
    split_store_colpart<E>(a, sh, acc_x, 2, vec, ok);
}

// ---------------------------------------------------------------- norm-free exit
// Backward of h = residual + dropout(x + bias) alone (no norm after it):
// dh = dh_out, so dx = keep ? dh_out * scale : 0, dbias = sum over rows of
// dx, and dresidual is dh_out itself (not written).  Tiles as the split
// path's second pass (tile_rows rows x one wave's 64 vectors, 4 waves taking
// rows w, w + 4, ..., U rows per group loaded ahead); the tile's dbias
// partial is added across the waves in wave order into slot 0 of its row
// block.
template <int U, int MW>
struct ExitIn {
    uint4 dho[U];
    uint32_t mask[U][MW];
};

template <typename IO, int DROP>
__global__ void __launch_bounds__(256) sp_region_bwd_exit_kernel(BwdArgs a) {
    using V = Vec<IO>;
    constexpr int E = V::N, U = kSplitUnroll, MW = E / 4;
    __shared__ float sh[kSplitWaves][64][E];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int vec = blockIdx.x * 64 + lane;
    const bool ok = vec < a.nvec;
    const int vcl = ok ? vec : a.nvec - 1;
    float acc[E];
#pragma unroll
    for (int j = 0; j < E; ++j) acc[j] = 0.0f;

    const int64_t r0 = (int64_t)blockIdx.y * a.tile_rows;
    const int64_t r1 = r0 + a.tile_rows < a.rows ? r0 + a.tile_rows : a.rows;
    constexpr int64_t step = kSplitWaves * U;

    auto load_group = [&](int64_t base, ExitIn<U, MW>& in) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + kSplitWaves * u;
            const int64_t rc = row < r1 ? row : r1 - 1;          // clamp: always a valid row
            const int64_t off = rc * a.hidden + (int64_t)vcl * E;
            in.dho[u] = load_stream(static_cast<const IO*>(a.dh_out) + off);
            if (DROP == kDropMask) {
#pragma unroll
                for (int w = 0; w < MW; ++w)
                    in.mask[u][w] = __builtin_nontemporal_load(
                        reinterpret_cast<const uint32_t*>(a.mask + off) + w);
            }
        }
    };

    ExitIn<U, MW> cur, nxt;
    int64_t base = r0 + wave;
    if (base < r1) load_group(base, cur);
    for (; base < r1; base += step) {
        if (base + step < r1) load_group(base + step, nxt);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + kSplitWaves * u;
            const bool rok = row < r1;                       // wave-uniform
            V dho, dx;
            dho.set(cur.dho[u]);
            uint32_t kb = 0xffu;
            if (DROP == kDropMask) {
                kb = MaskBytes<4>::from_word(cur.mask[u][0]);
                if (MW == 2) kb |= MaskBytes<4>::from_word(cur.mask[u][MW - 1]) << 4;
            } else if (DROP == kDropRegen) {
                kb = keep_bits<E>((a.row_base + (uint64_t)(rok ? row : r1 - 1)) *
                                          (uint64_t)a.hidden + (uint64_t)vcl * E,
                                  a.off_lo, a.off_hi, a.key_lo, a.key_hi, a.thr);
            }
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float dh = dho.v[j];
                const float dxu =
                    DROP != kDropNone ? (((kb >> j) & 1u) ? dh * a.scale : 0.0f) : dh;
                dx.v[j] = dxu;
                if (ok && rok) acc[j] += dxu;
            }
            if (ok && rok) dx.store(static_cast<IO*>(a.dx_out) + row * a.hidden + (int64_t)vec * E);
        }
        cur = nxt;
    }
    if (a.dbias_out) split_store_colpart<E>(a, sh, acc, 0, vec, ok);
}

static hipError_t launch_finalize(const BwdArgs& a, hipStream_t s);

hipError_t launch_bwd_exit(const spr_desc& d, const BwdPlan& p, const BwdArgs& a, hipStream_t s) {
    const dim3 g((unsigned)p.col_tiles, (unsigned)p.exit_row_blocks), b(256);
    const int mode = !(d.p > 0.0f) ? kDropNone : (a.mask ? kDropMask : kDropRegen);
    if (d.io == SPR_BF16) {
        if (mode == kDropMask)
            hipLaunchKernelGGL((sp_region_bwd_exit_kernel<__bf16, kDropMask>), g, b, 0, s, a);
        else if (mode == kDropRegen)
            hipLaunchKernelGGL((sp_region_bwd_exit_kernel<__bf16, kDropRegen>), g, b, 0, s, a);
        else
            hipLaunchKernelGGL((sp_region_bwd_exit_kernel<__bf16, kDropNone>), g, b, 0, s, a);
    } else {
        if (mode == kDropMask)
            hipLaunchKernelGGL((sp_region_bwd_exit_kernel<float, kDropMask>), g, b, 0, s, a);
        else if (mode == kDropRegen)
            hipLaunchKernelGGL((sp_region_bwd_exit_kernel<float, kDropRegen>), g, b, 0, s, a);
        else
            hipLaunchKernelGGL((sp_region_bwd_exit_kernel<float, kDropNone>), g, b, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.dbias_out) return e;
    return launch_finalize(a, s);
}

// Teams: one workgroup per CU (fewer workgroups cannot draw the full HBM
// bandwidth) and no more, since each team writes one partial row of 3*h fp32
// that the finalize reads back.
int64_t bwd_teams(const spr_desc& d, const RowPlan& p) {
    const int64_t rows = d.s_local * d.b;
    const int64_t cap = (int64_t)device_cu_count() * p.rpw;   // one workgroup per CU
    const int64_t want = rows < cap ? rows : cap;
    return ((want + p.rpw - 1) / p.rpw) * p.rpw;
}

template <typename IO, int NORM, int DROP, bool WR, bool EXACT>
static hipError_t bwd_by_vpt(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    const dim3 g((unsigned)(a.teams / p.rpw)), b((unsigned)p.block);
#define SPR_BWD_CASE(V, L)                                                                       \
    case V:                                                                                      \
        hipLaunchKernelGGL((sp_region_bwd_rows_kernel<IO, NORM, DROP, V, WR, L, EXACT>), g, b, 0, \
                           s, a);                                                                \
        break;
    if constexpr (WR) {
        switch (p.vpt) {
            SPR_BWD_CASE(1, 256) SPR_BWD_CASE(2, 256) SPR_BWD_CASE(3, 256) SPR_BWD_CASE(4, 256)
            default: return hipErrorInvalidValue;
        }
    } else {
        // must match kBwdCombos
        switch (p.vpt) {
            case 1:
                if (p.lb == 768) {
                    hipLaunchKernelGGL((sp_region_bwd_rows_kernel<IO, NORM, DROP, 1, WR, 768, EXACT>),
                                       g, b, 0, s, a);
                } else {
                    hipLaunchKernelGGL((sp_region_bwd_rows_kernel<IO, NORM, DROP, 1, WR, 1024, EXACT>),
                                       g, b, 0, s, a);
                }
                break;
            SPR_BWD_CASE(2, 768) SPR_BWD_CASE(3, 512)
            SPR_BWD_CASE(4, 512) SPR_BWD_CASE(5, 640) SPR_BWD_CASE(6, 512) SPR_BWD_CASE(8, 512)
            default: return hipErrorInvalidValue;
        }
    }
#undef SPR_BWD_CASE
    return hipGetLastError();
}

static hipError_t launch_finalize(const BwdArgs& a, hipStream_t s) {
    const int64_t n3 = (int64_t)a.slots * a.hidden;
    hipLaunchKernelGGL(sp_region_bwd_finalize_kernel, dim3((unsigned)((n3 + kFinCols - 1) / kFinCols)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename IO, int NORM, int DROP>
static hipError_t bwd_by_mode(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    const bool exact = p.nvec == p.vpt * p.tpr;
    if (p.rpw > 1)
        return exact ? bwd_by_vpt<IO, NORM, DROP, true, true>(p, a, s)
                     : bwd_by_vpt<IO, NORM, DROP, true, false>(p, a, s);
    return exact ? bwd_by_vpt<IO, NORM, DROP, false, true>(p, a, s)
                 : bwd_by_vpt<IO, NORM, DROP, false, false>(p, a, s);
}

template <typename IO, int NORM, bool WR, bool EXACT>
static hipError_t rowsum_by_vpt(const RowPlan& p, const BwdArgs& a, hipStream_t s) {
    const int64_t grid = WR ? (a.rows + p.rpw - 1) / p.rpw : a.rows;
    const dim3 g((unsigned)grid), b((unsigned)p.block);
#define SPR_RS_CASE(V, L)                                                                         \
    case V:                                                                                       \
        hipLaunchKernelGGL((sp_region_bwd_rowsum_kernel<IO, NORM, V, WR, L, EXACT>), g, b, 0, s, a); \
        break;
    if constexpr (WR) {
        switch (p.vpt) {
            SPR_RS_CASE(1, 256) SPR_RS_CASE(2, 256) SPR_RS_CASE(3, 256) SPR_RS_CASE(4, 256)
            default: return hipErrorInvalidValue;
        }
    } else {
        // must match kWgCombos (the forward's row plans)
        switch (p.vpt) {
            SPR_RS_CASE(1, 1024) SPR_RS_CASE(2, 1024) SPR_RS_CASE(3, 1024)
            SPR_RS_CASE(4, 1024) SPR_RS_CASE(5, 768) SPR_RS_CASE(6, 768) SPR_RS_CASE(8, 512)
            default: return hipErrorInvalidValue;
        }
    }
#undef SPR_RS_CASE
    return hipGetLastError();
}

template <typename IO, int NORM>
static hipError_t split_rowsum(const BwdPlan& p, const BwdArgs& a, hipStream_t s) {
    const RowPlan& rp = p.sum_rows;
    const bool exact = rp.nvec == rp.vpt * rp.tpr;
    if (rp.rpw > 1)
        return exact ? rowsum_by_vpt<IO, NORM, true, true>(rp, a, s)
                     : rowsum_by_vpt<IO, NORM, true, false>(rp, a, s);
    return exact ? rowsum_by_vpt<IO, NORM, false, true>(rp, a, s)
                 : rowsum_by_vpt<IO, NORM, false, false>(rp, a, s);
}

static int drop_mode(const spr_desc& d, const BwdArgs& a) {
    if (!(d.p > 0.0f)) return kDropNone;
    return a.mask ? kDropMask : kDropRegen;
}

template <typename IO, int NORM>
static hipError_t split_main(const spr_desc& d, const BwdPlan& p, const BwdArgs& a, hipStream_t s) {
    const dim3 g((unsigned)p.col_tiles, (unsigned)p.row_blocks), b(256);
    switch (drop_mode(d, a)) {
        case kDropMask:
            hipLaunchKernelGGL((sp_region_bwd_main_kernel<IO, NORM, kDropMask>), g, b, 0, s, a);
            break;
        case kDropRegen:
            hipLaunchKernelGGL((sp_region_bwd_main_kernel<IO, NORM, kDropRegen>), g, b, 0, s, a);
            break;
        default:
            hipLaunchKernelGGL((sp_region_bwd_main_kernel<IO, NORM, kDropNone>), g, b, 0, s, a);
    }
    return hipGetLastError();
}

template <typename IO, int NORM>
static hipError_t bwd_one(const spr_desc& d, const BwdPlan& p, const BwdArgs& a, hipStream_t s,
                          int index) {
    if (p.path == kBwdSplit) {
        if (index == 0) return split_rowsum<IO, NORM>(p, a, s);
        if (index == 1) return split_main<IO, NORM>(d, p, a, s);
        return launch_finalize(a, s);
    }
    if (index == 0) {
        switch (drop_mode(d, a)) {
            case kDropMask: return bwd_by_mode<IO, NORM, kDropMask>(p.rows, a, s);
            case kDropRegen: return bwd_by_mode<IO, NORM, kDropRegen>(p.rows, a, s);
            default: return bwd_by_mode<IO, NORM, kDropNone>(p.rows, a, s);
        }
    }
    return launch_finalize(a, s);
}

int bwd_num_launches(const BwdPlan& p) { return p.path == kBwdSplit ? 3 : 2; }

hipError_t launch_bwd(const spr_desc& d, const BwdPlan& p, const BwdArgs& a, hipStream_t s,
                      int first, int last) {
    for (int i = first; i < last; ++i) {
        hipError_t e;
        if (d.io == SPR_BF16)
            e = d.norm == SPR_LAYERNORM ? bwd_one<__bf16, SPR_LAYERNORM>(d, p, a, s, i)
                                        : bwd_one<__bf16, SPR_RMSNORM>(d, p, a, s, i);
        else
            e = d.norm == SPR_LAYERNORM ? bwd_one<float, SPR_LAYERNORM>(d, p, a, s, i)
                                        : bwd_one<float, SPR_RMSNORM>(d, p, a, s, i);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace spr
