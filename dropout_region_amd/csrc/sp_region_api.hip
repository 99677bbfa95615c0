// sp_region_api.hip -- the C ABI of include/sp_region.h: host-side argument
// checks, launch planning and dispatch.  Every check runs before the first
// HIP call, so an invalid call launches nothing and touches no output.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "sp_host_checks.h"
#include "sp_plan.h"
#include "sp_region.h"

namespace spr {

bool make_row_plan(int io, int64_t h, PlanKind kind, RowPlan* plan) {
    const int epv = (io == SPR_BF16) ? 8 : 4;
    if (h <= 0 || h % epv != 0) return false;
    const int64_t nvec = h / epv;
    RowPlan p{};
    p.epv = epv;
    p.nvec = (int)nvec;
    if (nvec <= 4 * 64) {                    // short rows: one wave per row, 4 rows per WG
        p.vpt = (int)((nvec + 63) / 64);
        p.tpr = 64;
        p.rpw = 4;
        p.block = 256;
        p.lb = 256;
        *plan = p;
        return true;
    }
    // One workgroup per row.  Take the first candidate (in preference order)
    // whose split leaves no vector slot idle, else the one wasting fewest.
    // The forward prefers more vectors per thread: more loads in flight per
    // thread and a smaller reduction (measured on MI355X, 22B shard: 6
    // vectors per thread 14.8 us, 4: 16.0, 3: 15.5, 2: 17.3).  The norm-only
    // entry, which loads half as much per element, is fastest at 4 (22B
    // shard: 8.0 us against 12.3 at 6).
    static const int kFwdOrder[] = {6, 4, 3, 5, 2, 8, 1};
    static const int kEntryOrder[] = {4, 3, 5, 6, 2, 8, 1};
    static const int kBwdOrder[] = {1, 2, 3, 4, 5, 6, 8};
    const bool fwd = kind != kPlanBackward;
    const int* order = kind == kPlanForward ? kFwdOrder : (kind == kPlanEntry ? kEntryOrder : kBwdOrder);
    int best_vpt = 0, best_lb = 0;
    int64_t best_tpr = 0, best_waste = INT64_MAX;
    for (int i = 0; i < 7; ++i) {
        const int v = order[i];
        const int64_t tpr = ((nvec + v - 1) / v + 63) / 64 * 64;
        const VptBound* tab = fwd ? kWgCombos : kBwdCombos;
        const int ntab = fwd ? (int)(sizeof kWgCombos / sizeof kWgCombos[0])
                             : (int)(sizeof kBwdCombos / sizeof kBwdCombos[0]);
        int lb = 0;                          // the smallest compiled bound that fits
        for (int t = 0; t < ntab; ++t)
            if (tab[t].vpt == v && tab[t].lb >= tpr && (lb == 0 || tab[t].lb < lb)) lb = tab[t].lb;
        if (lb == 0) continue;
        const int64_t waste = tpr * v - nvec;
        if (waste < best_waste) {
            best_waste = waste;
            best_vpt = v;
            best_lb = lb;
            best_tpr = tpr;
        }
    }
    if (best_vpt == 0) return false;
    p.vpt = best_vpt;
    p.tpr = (int)best_tpr;
    p.rpw = 1;
    p.block = p.tpr;
    p.lb = best_lb;
    *plan = p;
    return true;
}

// The dropout's generator key and counter words, threshold and scale, as
// both directions use them.  Element (r, c) of the shard is element
// e = (shard_index*N + r)*h + c of the full tensor.
template <typename Args>
static void set_dropout(const spr_desc& d, int64_t rows, Args* a) {
    a->row_base = (uint64_t)d.shard_index * (uint64_t)rows;
    a->key_lo = (uint32_t)d.seed;
    a->key_hi = (uint32_t)(d.seed >> 32);
    a->off_lo = (uint32_t)d.offset;
    a->off_hi = (uint32_t)(d.offset >> 32);
    // keep iff word >= floor(p * 2^32); p * 2^32 is exact in double
    a->thr = (uint32_t)floor((double)d.p * 4294967296.0);
    a->scale = (float)(1.0 / (1.0 - (double)d.p));
}

bool make_stream_plan(int io, int64_t h, RowPlan* plan) {
    const int epv = (io == SPR_BF16) ? 8 : 4;
    if (h <= 0 || h % epv != 0) return false;
    const int64_t nvec = h / epv;
    if (nvec <= 4 * 64) return false;        // one wave per row instead
    // Most vectors per thread first (more bytes in flight per thread); the
    // first split with no idle slot, else the one with the fewest.
    const int max_vpt = 16 / epv;
    int best_vpt = 0;
    int64_t best_tpr = 0, best_waste = INT64_MAX;
    for (int v = max_vpt; v >= 1; --v) {
        const int64_t tpr = ((nvec + v - 1) / v + 63) / 64 * 64;
        if (tpr > stream_bound(epv, v)) continue;
        const int64_t waste = tpr * v - nvec;
        if (waste < best_waste) {
            best_waste = waste;
            best_vpt = v;
            best_tpr = tpr;
        }
    }
    if (best_vpt == 0) return false;
    RowPlan p{};
    p.epv = epv;
    p.nvec = (int)nvec;
    p.vpt = best_vpt;
    p.tpr = (int)best_tpr;
    p.rpw = 1;
    p.block = p.tpr;
    p.lb = stream_bound(epv, best_vpt);
    *plan = p;
    return true;
}

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cus[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1) {
            (void)hipGetLastError();
            n = 256;
        }
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

static size_t round256(uint64_t b) { return (size_t)((b + 255u) & ~(uint64_t)255u); }

// Chooses the backward path: fused whenever its row team fits in registers
// (at most two vectors per thread), split otherwise -- measured on MI355X,
// the fused path is the faster one wherever it applies, even on shards where
// its partial rows outweigh the split path's second read of dy and h.
// desc.bwd_path asks for one path, desc.bwd_tile_rows for a tile height.
bool make_bwd_plan(const spr_desc& d, BwdPlan* plan) {
    BwdPlan p{};
    if (!make_row_plan(d.io, d.h, kPlanBackward, &p.rows)) return false;
    if (!make_row_plan(d.io, d.h, kPlanForward, &p.sum_rows)) return false;
    const int64_t rows = d.s_local * d.b;
    const bool fused_ok = p.rows.vpt <= 2;
    p.teams = bwd_teams(d, p.rows);

    p.col_tiles = (p.rows.nvec + 63) / 64;
    // Rows per tile, a multiple of the 16 rows a workgroup's four waves take
    // per group: 32 for the split path's second pass, 16 for the exit.  Many
    // small tiles keep several workgroups per CU loading at once, and the
    // partial rows they add stay a few % of the bytes (3*h fp32 per tile row
    // against 9 bytes per element in, 1*h against 5).  Measured on MI355X
    // against about one tile per CU: split second pass + finalize 61.6 ->
    // 47.7 us on the 175B shard, 358 -> 328 us on the 1T t = 1 shard; exit
    // 33.4 -> 27.4 us (175B), 194 -> 176 us (1T t = 1).
    // desc.bwd_tile_rows (a multiple of 16) overrides both.
    const int64_t rows16 = (rows + 15) / 16 * 16;
    int64_t tr = 32, tr_exit = 16;
    if (d.bwd_tile_rows > 0) tr = tr_exit = d.bwd_tile_rows;
    // The row blocks are the grid's y dimension, at most 65535.
    const int64_t min_tr = ((rows + 65534) / 65535 + 15) / 16 * 16;
    if (tr < min_tr) tr = min_tr;
    if (tr_exit < min_tr) tr_exit = min_tr;
    if (tr > rows16) tr = rows16;
    if (tr_exit > rows16) tr_exit = rows16;
    p.tile_rows = (int)tr;
    p.row_blocks = (rows + tr - 1) / tr;
    p.exit_tile_rows = (int)tr_exit;
    p.exit_row_blocks = (rows + tr_exit - 1) / tr_exit;
    p.rowpart_bytes = round256((uint64_t)rows * 2u * sizeof(float));

    p.path = fused_ok ? kBwdFused : kBwdSplit;
    if (d.bwd_path == SPR_BWD_SPLIT) p.path = kBwdSplit;

    const uint64_t fused_ws = (uint64_t)p.teams * 3u * (uint64_t)d.h * sizeof(float);
    const uint64_t split_ws = p.rowpart_bytes + (uint64_t)p.row_blocks * 3u * (uint64_t)d.h * sizeof(float);
    const uint64_t exit_ws = (uint64_t)p.exit_row_blocks * (uint64_t)d.h * sizeof(float);
    p.bwd_workspace = round256(p.path == kBwdFused ? fused_ws : split_ws);
    p.workspace = p.bwd_workspace > round256(exit_ws) ? p.bwd_workspace : round256(exit_ws);
    *plan = p;
    return true;
}

}  // namespace spr

using namespace spr;

namespace {

// Field checks shared by every entry point.
spr_status check_fields(const spr_desc* d) {
    if (!d) return SPR_ERR_INVALID_ARG;
    if (d->s_local < 1 || d->b < 1 || d->h < 1) return SPR_ERR_INVALID_ARG;
    if (d->t < 1 || d->shard_index < 0 || d->shard_index >= d->t) return SPR_ERR_INVALID_ARG;
    if (d->io != SPR_F32 && d->io != SPR_BF16) return SPR_ERR_INVALID_ARG;
    if (d->norm != SPR_LAYERNORM && d->norm != SPR_RMSNORM) return SPR_ERR_INVALID_ARG;
    if (!(d->p >= 0.0f && d->p < 1.0f)) return SPR_ERR_INVALID_ARG;      // also rejects NaN
    if (!(d->eps > 0.0f) || isinf(d->eps)) return SPR_ERR_INVALID_ARG;
    if (d->fwd_kernel < SPR_FWD_AUTO || d->fwd_kernel > SPR_FWD_STREAM) return SPR_ERR_INVALID_ARG;
    if (d->bwd_path < SPR_BWD_AUTO || d->bwd_path > SPR_BWD_SPLIT) return SPR_ERR_INVALID_ARG;
    if (d->bwd_tile_rows != 0 &&
        (d->bwd_tile_rows < 16 || d->bwd_tile_rows % 16 != 0 || d->bwd_tile_rows > (1 << 20)))
        return SPR_ERR_INVALID_ARG;
    if (d->reserved != 0) return SPR_ERR_INVALID_ARG;
    // N*h and the global element index (t*N*h) must fit comfortably in 63 bits.
    if (d->s_local > (INT64_C(1) << 40) / d->b) return SPR_ERR_UNSUPPORTED;
    const int64_t rows = d->s_local * d->b;
    if ((double)rows * (double)d->h * (double)d->t > 9.0e18) return SPR_ERR_UNSUPPORTED;
    return SPR_OK;
}

// Field checks plus what the kernels handle; fills the launch plan.
spr_status check_desc(const spr_desc* d, RowPlan* plan, PlanKind kind) {
    const spr_status st = check_fields(d);
    if (st != SPR_OK) return st;
    if (d->s_local * d->b > INT32_MAX) return SPR_ERR_UNSUPPORTED;
    if (d->h / (d->io == SPR_BF16 ? 8 : 4) > 4096) return SPR_ERR_UNSUPPORTED;
    if (!make_row_plan(d->io, d->h, kind, plan)) return SPR_ERR_UNSUPPORTED;
    return SPR_OK;
}

}  // namespace

namespace {

constexpr int32_t kMaxParts = 1024;

// Every check of the forward, then the launch.  x holds nparts slabs of
// [N, h] (nparts == 1: the plain forward).
spr_status fwd_impl(const spr_desc* d, const void* x, int nparts, const float* bias,
                    const void* residual, const float* gamma, const float* beta, void* h_out,
                    void* y_out, uint8_t* mask_out, float* mean_out, float* rstd_out,
                    hipStream_t stream) {
    RowPlan plan;
    spr_status st = check_desc(d, &plan, x ? kPlanForward : kPlanEntry);
    if (st != SPR_OK) return st;
    const bool ln = d->norm == SPR_LAYERNORM, drop = d->p > 0.0f;
    if (!residual || (!x && !gamma)) return SPR_ERR_INVALID_ARG;
    if (x) {                             // the branch: x (+ bias), dropout, residual add
        if (!h_out) return SPR_ERR_INVALID_ARG;
    } else {                             // norm-only entry: h is the residual
        if (drop || bias || nparts != 1) return SPR_ERR_INVALID_ARG;
    }
    if (gamma) {                         // the norm
        if (!y_out || !rstd_out) return SPR_ERR_INVALID_ARG;
        if (ln != (beta != nullptr) || ln != (mean_out != nullptr)) return SPR_ERR_INVALID_ARG;
    } else {                             // norm-free exit: h and the mask only
        if (beta || y_out || mean_out || rstd_out) return SPR_ERR_INVALID_ARG;
    }
    if (!drop) mask_out = nullptr;                                   // ignored at p == 0
    const void* io16[] = {x, residual, h_out, y_out};
    for (const void* p : io16)
        if (!aligned(p, 16)) return SPR_ERR_INVALID_ARG;
    if (!aligned(bias, 16) || !aligned(gamma, 16) || !aligned(beta, 16)) return SPR_ERR_INVALID_ARG;
    if (!aligned(mask_out, 8) || !aligned(mean_out, 4) || !aligned(rstd_out, 4))
        return SPR_ERR_INVALID_ARG;

    const int64_t rows = d->s_local * d->b;
    const uint64_t E = (uint64_t)rows * (uint64_t)d->h;
    const uint64_t es = (d->io == SPR_BF16) ? 2u : 4u;
    const uint64_t pb = (uint64_t)d->h * 4u, sb = (uint64_t)rows * 4u;
    const Range outs[] = {range_of(h_out, E * es), range_of(y_out, E * es), range_of(mask_out, E),
                          range_of(mean_out, sb), range_of(rstd_out, sb)};
    const Range ins[] = {range_of(x, (uint64_t)nparts * E * es), range_of(residual, E * es),
                         range_of(bias, pb),
                         range_of(gamma, pb), range_of(beta, pb)};
    if (!disjoint(outs, 5, ins, 5)) return SPR_ERR_INVALID_ARG;

    FwdArgs a{};
    a.x = x; a.bias = bias; a.residual = residual; a.gamma = gamma; a.beta = beta;
    a.h_out = h_out; a.y_out = y_out; a.mask_out = mask_out; a.mean_out = mean_out;
    a.rstd_out = rstd_out;
    a.rows = rows;
    a.hidden = d->h;
    set_dropout(*d, rows, &a);
    a.inv_h = (float)(1.0 / (double)d->h);
    a.eps = d->eps;
    a.nvec = plan.nvec;
    a.nparts = nparts;
    a.part_stride = (int64_t)E;
    return launch_fwd(*d, plan, a, stream) == hipSuccess ? SPR_OK : SPR_ERR_HIP;
}

}  // namespace

extern "C" {

const char* sp_region_status_string(int s) {
    switch (s) {
        case SPR_OK: return "ok";
        case SPR_ERR_INVALID_ARG: return "invalid argument";
        case SPR_ERR_UNSUPPORTED: return "unsupported shape";
        case SPR_ERR_WORKSPACE: return "workspace missing or too small";
        case SPR_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

spr_status sp_region_activation_bytes(const spr_desc* d, uint64_t* saved_for_bwd,
                                      uint64_t* retained_output) {
    const spr_status st = check_fields(d);
    if (st != SPR_OK) return st;
    if (!saved_for_bwd || !retained_output) return SPR_ERR_INVALID_ARG;
    const uint64_t rows = (uint64_t)(d->s_local * d->b);
    const uint64_t elems = rows * (uint64_t)d->h;
    const uint64_t io_bytes = (d->io == SPR_BF16) ? 2u : 4u;
    const uint64_t h_bytes = elems * io_bytes;                       // the norm input h
    const uint64_t mask = (d->p > 0.0f) ? elems : 0u;                // 1 byte per element
    const uint64_t stats = rows * ((d->norm == SPR_LAYERNORM) ? 2u : 1u) * sizeof(float);
    *saved_for_bwd = h_bytes + mask + stats;
    *retained_output = elems * io_bytes;                             // y, the next block's input
    return SPR_OK;
}

size_t sp_region_bwd_workspace_bytes(const spr_desc* d) {
    RowPlan rp;
    BwdPlan plan;
    if (check_desc(d, &rp, kPlanBackward) != SPR_OK || !make_bwd_plan(*d, &plan)) return 0;
    return plan.workspace;
}

spr_status sp_region_fwd(const spr_desc* d, const void* x, const float* bias,
                         const void* residual, const float* gamma, const float* beta,
                         void* h_out, void* y_out, uint8_t* mask_out, float* mean_out,
                         float* rstd_out, hipStream_t stream) {
    return fwd_impl(d, x, 1, bias, residual, gamma, beta, h_out, y_out, mask_out, mean_out,
                    rstd_out, stream);
}

spr_status sp_region_fwd_rs(const spr_desc* d, const void* x_parts, int32_t nparts,
                            const float* bias, const void* residual, const float* gamma,
                            const float* beta, void* h_out, void* y_out, uint8_t* mask_out,
                            float* mean_out, float* rstd_out, hipStream_t stream) {
    if (!x_parts || nparts < 1 || nparts > kMaxParts) return SPR_ERR_INVALID_ARG;
    return fwd_impl(d, x_parts, nparts, bias, residual, gamma, beta, h_out, y_out, mask_out,
                    mean_out, rstd_out, stream);
}

}  // extern "C"

namespace {

// The backward's workspace in the kernel arguments: the split path's per-row
// sums first, then the column partials.
void set_workspace(const BwdPlan& plan, void* workspace, BwdArgs* a) {
    const bool split = plan.path == kBwdSplit;
    a->rowpart = static_cast<float*>(workspace);
    a->partials = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           (split ? plan.rowpart_bytes : 0));
}

// Every check of the backward, then the kernel arguments and plan.  With
// fixed_scratch the workspace is the library's own array (set afterwards):
// only its size is checked.
spr_status prepare_bwd(const spr_desc* d, const void* dy, const void* dh_out, const void* h,
                       const uint8_t* mask, const float* mean, const float* rstd,
                       const float* gamma, void* dx_out, void* dres_out, float* dgamma_out,
                       float* dbeta_out, float* dbias_out, void* workspace,
                       size_t workspace_bytes_given, BwdPlan* plan_out, BwdArgs* args_out,
                       bool fixed_scratch = false) {
    RowPlan rp;
    spr_status st = check_desc(d, &rp, kPlanBackward);
    if (st != SPR_OK) return st;
    BwdPlan plan;
    if (!make_bwd_plan(*d, &plan)) return SPR_ERR_UNSUPPORTED;
    const bool ln = d->norm == SPR_LAYERNORM, drop = d->p > 0.0f;
    if (!dy || !h || !rstd || !gamma || !dres_out || !dgamma_out)   // dx_out: optional
        return SPR_ERR_INVALID_ARG;
    if (ln != (mean != nullptr) || ln != (dbeta_out != nullptr)) return SPR_ERR_INVALID_ARG;
    if (!drop) mask = nullptr;          // p > 0 without a mask: regenerated
    const void* io16[] = {dy, dh_out, h, dx_out, dres_out, gamma};
    for (const void* p : io16)
        if (!aligned(p, 16)) return SPR_ERR_INVALID_ARG;
    if (!aligned(mask, 8) || !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(dgamma_out, 4) ||
        !aligned(dbeta_out, 4) || !aligned(dbias_out, 4))
        return SPR_ERR_INVALID_ARG;
    const size_t need = plan.bwd_workspace;
    if (fixed_scratch) {
        if (need > workspace_bytes_given) return SPR_ERR_WORKSPACE;
        workspace = nullptr;
    } else if (!workspace || workspace_bytes_given < need || !aligned(workspace, 16)) {
        return SPR_ERR_WORKSPACE;
    }

    const int64_t rows = d->s_local * d->b;
    const uint64_t E = (uint64_t)rows * (uint64_t)d->h;
    const uint64_t es = (d->io == SPR_BF16) ? 2u : 4u;
    const uint64_t pb = (uint64_t)d->h * 4u, sb = (uint64_t)rows * 4u;
    const Range outs[] = {range_of(dx_out, E * es), range_of(dres_out, E * es),
                          range_of(dgamma_out, pb), range_of(dbeta_out, pb),
                          range_of(dbias_out, pb), range_of(workspace, need)};
    const Range ins[] = {range_of(dy, E * es), range_of(dh_out, E * es), range_of(h, E * es),
                         range_of(mask, E), range_of(mean, sb), range_of(rstd, sb),
                         range_of(gamma, pb)};
    if (!disjoint(outs, 6, ins, 7)) return SPR_ERR_INVALID_ARG;

    BwdArgs a{};
    a.dy = dy; a.dh_out = dh_out; a.h = h; a.mask = mask; a.mean = mean; a.rstd = rstd;
    a.gamma = gamma; a.dx_out = dx_out; a.dres_out = dres_out;
    const bool split = plan.path == kBwdSplit;
    set_workspace(plan, workspace, &a);
    a.dgamma_out = dgamma_out; a.dbeta_out = dbeta_out; a.dbias_out = dbias_out;
    a.rows = rows;
    a.hidden = d->h;
    set_dropout(*d, rows, &a);
    a.inv_h = (float)(1.0 / (double)d->h);
    a.nvec = plan.rows.nvec;
    a.teams = (int)(split ? plan.row_blocks : plan.teams);
    a.col_tiles = plan.col_tiles;
    a.tile_rows = plan.tile_rows;
    a.slots = 3;
    *plan_out = plan;
    *args_out = a;
    return SPR_OK;
}

}  // namespace

extern "C" {

spr_status sp_region_bwd(const spr_desc* d, const void* dy, const void* dh_out, const void* h,
                         const uint8_t* mask, const float* mean, const float* rstd,
                         const float* gamma, void* dx_out, void* dres_out, float* dgamma_out,
                         float* dbeta_out, float* dbias_out, void* workspace,
                         size_t workspace_bytes_given, hipStream_t stream) {
    BwdPlan plan;
    BwdArgs a;
    const spr_status st = prepare_bwd(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out,
                                      dgamma_out, dbeta_out, dbias_out, workspace,
                                      workspace_bytes_given, &plan, &a);
    if (st != SPR_OK) return st;
    return launch_bwd(*d, plan, a, stream, 0, bwd_num_launches(plan)) == hipSuccess ? SPR_OK
                                                                                    : SPR_ERR_HIP;
}

}  // extern "C"

namespace {

// The allocation-free backward's scratch: one fixed array per GPU, in this
// library's device memory.  Host code never passes `scratch` itself to a
// kernel (on the host the name is only a stand-in for the symbol); it
// passes the device address hipGetSymbolAddress gives, looked up once per
// device and kept.
static __device__ __align__(256) unsigned char scratch[SPR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> scratch_ptr[kMaxScratchDevices];

// The current device's address of `scratch`, or NULL if it cannot be had.
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

spr_status sp_region_bwd_noalloc(const spr_desc* d, const void* dy, const void* dh_out,
                                 const void* h, const uint8_t* mask, const float* mean,
                                 const float* rstd, const float* gamma, void* dx_out,
                                 void* dres_out, float* dgamma_out, float* dbeta_out,
                                 float* dbias_out, hipStream_t stream) {
    BwdPlan plan;
    BwdArgs a;
    const spr_status st = prepare_bwd(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out,
                                      dgamma_out, dbeta_out, dbias_out, nullptr,
                                      SPR_NOALLOC_SCRATCH_BYTES, &plan, &a, true);
    if (st != SPR_OK) return st;
    void* ws = scratch_address();
    if (!ws) return SPR_ERR_HIP;
    set_workspace(plan, ws, &a);
    return launch_bwd(*d, plan, a, stream, 0, bwd_num_launches(plan)) == hipSuccess ? SPR_OK
                                                                                    : SPR_ERR_HIP;
}

int sp_region_bwd_num_launches(const spr_desc* d) {
    RowPlan rp;
    BwdPlan plan;
    if (check_desc(d, &rp, kPlanBackward) != SPR_OK || !make_bwd_plan(*d, &plan)) return 0;
    return bwd_num_launches(plan);
}

spr_status sp_region_bwd_launch(const spr_desc* d, int index, const void* dy, const void* dh_out,
                                const void* h, const uint8_t* mask, const float* mean,
                                const float* rstd, const float* gamma, void* dx_out,
                                void* dres_out, float* dgamma_out, float* dbeta_out,
                                float* dbias_out, void* workspace, size_t workspace_bytes_given,
                                hipStream_t stream) {
    BwdPlan plan;
    BwdArgs a;
    const spr_status st = prepare_bwd(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out,
                                      dgamma_out, dbeta_out, dbias_out, workspace,
                                      workspace_bytes_given, &plan, &a);
    if (st != SPR_OK) return st;
    if (index < 0 || index >= bwd_num_launches(plan)) return SPR_ERR_INVALID_ARG;
    return launch_bwd(*d, plan, a, stream, index, index + 1) == hipSuccess ? SPR_OK : SPR_ERR_HIP;
}

spr_status sp_region_bwd_exit(const spr_desc* d, const void* dh_out, const uint8_t* mask,
                              void* dx_out, float* dbias_out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    RowPlan rp;
    spr_status st = check_desc(d, &rp, kPlanBackward);
    if (st != SPR_OK) return st;
    BwdPlan plan;
    if (!make_bwd_plan(*d, &plan)) return SPR_ERR_UNSUPPORTED;
    if (!dh_out || !dx_out) return SPR_ERR_INVALID_ARG;
    if (!(d->p > 0.0f)) mask = nullptr;
    if (!aligned(dh_out, 16) || !aligned(dx_out, 16) || !aligned(mask, 8) ||
        !aligned(dbias_out, 4))
        return SPR_ERR_INVALID_ARG;
    const int64_t rows = d->s_local * d->b;
    const uint64_t E = (uint64_t)rows * (uint64_t)d->h;
    const uint64_t es = (d->io == SPR_BF16) ? 2u : 4u;
    // slot 0 of [row_blocks][1][h] fp32 column partials
    const size_t need = dbias_out ? (size_t)plan.exit_row_blocks * (size_t)d->h * sizeof(float) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return SPR_ERR_WORKSPACE;
    const Range outs[] = {range_of(dx_out, E * es), range_of(dbias_out, (uint64_t)d->h * 4u),
                          range_of(need ? workspace : nullptr, need)};
    const Range ins[] = {range_of(dh_out, E * es), range_of(mask, E)};
    if (!disjoint(outs, 3, ins, 2)) return SPR_ERR_INVALID_ARG;

    BwdArgs a{};
    a.dh_out = dh_out; a.mask = mask; a.dx_out = dx_out; a.dbias_out = dbias_out;
    a.partials = static_cast<float*>(workspace);
    a.rows = rows;
    a.hidden = d->h;
    set_dropout(*d, rows, &a);
    a.nvec = plan.rows.nvec;
    a.teams = (int)plan.exit_row_blocks;
    a.col_tiles = plan.col_tiles;
    a.tile_rows = plan.exit_tile_rows;
    a.slots = 1;
    return launch_bwd_exit(*d, plan, a, stream) == hipSuccess ? SPR_OK : SPR_ERR_HIP;
}

}  // extern "C"
