// sp_plan.h -- launch plans and kernel argument blocks (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sp_region.h"

namespace spr {

// How one row of h elements is spread over threads.  A row is cut into
// 16-byte vectors (8 bf16 or 4 fp32 elements); thread `tid` of the row's
// team owns vectors tid, tid + tpr, ..., tid + (vpt-1)*tpr, so each load
// instruction of a wave covers 1 KiB of contiguous memory.
struct RowPlan {
    int epv;        // elements per vector (8 bf16, 4 fp32)
    int nvec;       // vectors per row, h / epv
    int vpt;        // vectors per thread (compile-time in the kernels)
    int tpr;        // threads per row team (multiple of 64)
    int rpw;        // row teams per workgroup (4 one-wave teams, or 1)
    int block;      // threads per workgroup = tpr * rpw
    int lb;         // the kernel's launch bound (>= block): caps VGPRs per wave
};

// The (vectors per thread, launch bound) pairs compiled for whole-workgroup
// rows.  A bound of 1024 threads leaves 128 VGPRs per wave, 768 leaves 168,
// 512 leaves 256; more vectors per thread need more registers.
struct VptBound {
    int vpt, lb;
};
static constexpr VptBound kWgCombos[] = {{1, 1024}, {2, 1024}, {3, 1024}, {4, 1024},
                                         {5, 768},  {6, 768},  {8, 512}};
// The backward runs one workgroup per CU and keeps three column accumulators
// per element and DEPTH rows in flight in registers, so its bound tracks the
// workgroup it needs.  One vector per thread has two bounds: 768 threads
// leave room for three rows in flight, 1024 threads (rows of up to 1024
// vectors) for two.  A plan takes the smallest bound that fits its team.
static constexpr VptBound kBwdCombos[] = {{1, 768}, {1, 1024}, {2, 768}, {3, 512},
                                          {4, 512}, {5, 640},  {6, 512}, {8, 512}};

// Rows in flight per thread in the backward's row kernel (measured on
// MI355X): one vector per thread -> three rows (two at 1024 threads with
// LayerNorm, where a third would spill), two vectors -> none ahead (a
// prefetch row spills at 768 threads and was slower even at one ahead),
// wider rows -> none.  Short one-wave rows keep one row ahead.
constexpr int bwd_depth(int vpt, int lb, bool wave_rows, bool layernorm) {
    return wave_rows ? (vpt <= 2 ? 2 : 1)
                     : (vpt == 1 ? ((lb <= 768 || !layernorm) ? 3 : 2) : 1);
}

// Forward, the forward's norm-only entry (x absent: residual in, y out), or
// the backward: each has its own preference of vectors per thread.
enum PlanKind { kPlanForward, kPlanEntry, kPlanBackward };

// How the backward learns the dropout decisions: none (p == 0), from the
// stored mask, or regenerated from the counter-based generator (the forward
// stored no mask).
enum DropMode { kDropNone = 0, kDropMask = 1, kDropRegen = 2 };

// Launch bound of the forward's stream kernel for VPT vectors of E
// elements per thread: 1024 threads (128 VGPRs) up to 8 elements, 768 (168)
// up to 12, else 512 (256).
constexpr int stream_bound(int e, int vpt) {
    return e * vpt <= 8 ? 1024 : (e * vpt <= 12 ? 768 : 512);
}
// Row plan of the forward's stream kernel (one workgroup per row team, at
// most 16 elements per thread); false where it does not apply (short rows,
// which go one wave per row, and wide rows).
bool make_stream_plan(int io, int64_t h, RowPlan* plan);

// Picks a row plan for h; false if h is unsupported.  The forward prefers
// about four vectors per thread, the backward (which keeps three column
// accumulators per element) as few as possible.
bool make_row_plan(int io, int64_t h, PlanKind kind, RowPlan* plan);

struct FwdArgs {
    const void* x;
    const float* bias;
    const void* residual;
    const float* gamma;
    const float* beta;
    void* h_out;
    void* y_out;
    uint8_t* mask_out;
    float* mean_out;
    float* rstd_out;
    int64_t rows;          // N
    int64_t hidden;        // h
    uint64_t row_base;     // shard_index * N: global index of this shard's row 0
    uint32_t key_lo, key_hi, off_lo, off_hi;
    uint32_t thr;          // floor(p * 2^32)
    float scale;           // fp32(1 / (1 - p))
    float inv_h;           // 1 / h
    float eps;
    int nvec;
    int nparts;            // > 1: x holds nparts partial slabs, summed in the kernel
    int64_t part_stride;   // elements between two slabs (N * h)
};

struct BwdArgs {
    const void* dy;
    const void* dh_out;
    const void* h;
    const uint8_t* mask;
    const float* mean;
    const float* rstd;
    const float* gamma;
    void* dx_out;
    void* dres_out;
    float* partials;       // [teams][3][h] fp32 column partials (split path: [row_blocks][3][h])
    float* rowpart;        // split path: [N] float2 row sums (sum g, sum g*xhat)
    float* dgamma_out;
    float* dbeta_out;
    float* dbias_out;
    int64_t rows;
    int64_t hidden;
    uint64_t row_base;     // shard_index * N (regenerated dropout only)
    uint32_t key_lo, key_hi, off_lo, off_hi;
    uint32_t thr;
    float scale;
    float inv_h;
    int nvec;
    int teams;             // row teams in the grid = partial rows
    int col_tiles;         // split path: tiles of one wave's 64 vectors across a row
    int tile_rows;         // split path: rows per tile
    int slots;             // partial rows per team: 3 (dgamma, dbeta, dbias) or 1 (dbias)
};

// The backward's two strategies.
//  fused: one persistent workgroup per CU owns whole rows; its register column
//         partials make one partial row of 3*h fp32 per workgroup.
//  split: a read-only pass over dy and h gives each row its two sums; a
//         second pass over column tiles writes dx, dresidual and the
//         dgamma/dbeta/dbias partials of its rows.
enum BwdPath { kBwdFused = 0, kBwdSplit = 1 };

struct BwdPlan {
    RowPlan rows;          // fused: the row-team plan
    RowPlan sum_rows;      // split: the row plan of the row-sum pass (the forward's)
    int path;
    int64_t teams;         // fused: partial rows
    int col_tiles;         // split
    int tile_rows;         // split
    int64_t row_blocks;    // split: partial rows
    int exit_tile_rows;    // norm-free exit: rows per tile
    int64_t exit_row_blocks;  // norm-free exit: partial rows
    size_t rowpart_bytes;  // split: offset of the column partials in the workspace
    size_t bwd_workspace;  // bytes the chosen backward path needs
    size_t workspace;      // bytes the backward or the norm-free exit needs (the larger)
};

bool make_bwd_plan(const spr_desc& d, BwdPlan* plan);

// Compute units of the current device, queried once per device and kept
// (a launch fact, like an occupancy).  Where no device can be queried (a
// process without a GPU sizing a workspace) it is the 256 of a whole
// MI355X, the chip this library is built for.
int device_cu_count();

// Kernel launches of the backward for this plan (fused: rows, finalize;
// split: rowsum, main, finalize).
int bwd_num_launches(const BwdPlan& plan);

hipError_t launch_fwd(const spr_desc& d, const RowPlan& plan, const FwdArgs& a, hipStream_t s);

// Number of row teams (= fp32 partial rows) the fused backward uses.
int64_t bwd_teams(const spr_desc& d, const RowPlan& plan);
// The norm-free exit's backward: dx = keep ? dh_out * scale : 0 over the
// split path's tiles, then (with dbias) the finalize over one slot.
hipError_t launch_bwd_exit(const spr_desc& d, const BwdPlan& plan, const BwdArgs& a,
                           hipStream_t s);
// Runs launches [first, last) of the backward's sequence.
hipError_t launch_bwd(const spr_desc& d, const BwdPlan& plan, const BwdArgs& a, hipStream_t s,
                      int first, int last);

}  // namespace spr
