// ring_attn.hip -- one rank's ring-attention forward on gfx950 (context
// parallelism).
//
// Context parallelism gives rank i a contiguous block of query tokens and the
// matching K/V block; ring attention passes the K/V blocks around the ring
// and, at each step, attends the rank's queries to the block in hand and
// accumulates the partial online-softmax result, so that after t steps every
// query has attended every key and no device holds more than an s/t x s/t
// tile of scores ("Sequence parallel math", section "Context parallelism and
// ring attention").  No causal mask: every query sees every key.
//
// Kernel 1 (step): one workgroup of eight waves per (256-query tile,
// batch x head, group of consecutive ring steps), on a one-dimensional grid
// ordered so that the tiles streaming the same K/V blocks share an XCD; at
// step k the block in hand is block (rank - k) mod t.  It walks the blocks of
// its steps in ring order as one run of 64-key tiles with an online softmax
// and writes the group's partial result: O normalised by its own sum, and its
// log-sum-exp.  (One step per workgroup when the steps arrive one at a time;
// the fused call groups them so that about one workgroup per CU remains.)
// Kernel 2 (merge): per query and head, folds the partials in ring order,
// acc = merge(acc, partial_k) -- the accumulation a ring performs as the
// blocks arrive.
//
// Matrix products on MFMA (v_mfma_f32_32x32x16_bf16; bf16 operands, fp32
// accumulation).  Each wave owns 32 queries and computes S^T = K Q^T, so a
// lane holds the scores of ONE query (lane mod 32) for 32 of a tile's 64
// keys; the row max and sum need one exchange between the two half-waves.
// P (bf16) then feeds O^T += V^T P^T straight from registers, with the keys
// of each product taken in the order the score layout left them in (the
// same order for V^T, read from a transposed V tile in LDS), and O^T keeps
// one query per lane too, so the softmax rescale is one scalar per lane.
#include <hip/hip_runtime.h>
#include <math.h>

#include <atomic>

#include "sp_device.h"
#include "sp_host_checks.h"
#include "sp_plan.h"
#include "sp_ring_attn.h"

namespace spr {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

struct AttnArgs {
    const __bf16* q;       // [s_local][b][heads][d]
    const __bf16* k;       // fused: [t][s_local][b][heads][d]; one step: the block in hand
    const __bf16* v;
    float* part_o;         // [t][s_local][b][heads][d] fp32, normalised per step
    float* part_lse;       // [t][s_local][b][heads] fp32 (natural log)
    __bf16* o_out;         // [s_local][b][heads][d]
    float* lse_out;        // [s_local][b][heads]
    int64_t s_local, b;
    int heads, t, rank;
    int step0;             // ring step of the first step in the grid (one-step calls)
    int fused;             // 1: k/v hold all t blocks, block (rank - step) mod t is used
    int spg;               // ring steps per workgroup, walked as one run of key tiles
    int nparts;            // partial results the merge folds, in ring order
    float scale_log2;      // softmax scale * log2(e): scores in base-2 units
};

constexpr int kKT = 64;    // keys per tile
constexpr int kWaves = 8;  // waves per workgroup: 32 queries each
constexpr float kStale = 8.0f;   // base-2 headroom before the softmax reference moves

// The transposed V tile [d][column] stores key vpos(j) in column j: bits 2
// and 3 of the key index are swapped (the map is its own inverse).  The eight
// keys one lane feeds into an O^T product, {4g..4g+3, 8+4g..8+4g+3} of a
// 16-key group, then sit in eight adjacent columns: one 16-byte read.
__device__ __forceinline__ constexpr int vpos(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}
// Column swizzle: row d keeps its columns XOR-ed with vswz(d), a multiple of
// 8 (the 16-byte read groups stay whole).  It spreads the 16 rows that one
// staging write's lanes fill, and the rows 32 reading lanes cover, over
// distinct LDS banks.
__device__ __forceinline__ int vswz(int row) { return 8 * ((row >> 4) & 7); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// W waves of 32 queries each share every staged K/V tile (W * 32 queries
// per workgroup); two waves per SIMD either way (4 waves: two workgroups per
// CU, 8 waves: one).
// RUN: the workgroup walks a.spg > 1 ring steps as one run of key tiles;
// without it, one step (a.spg == 1) and no block changes inside the loop.
template <int D, int W, bool RUN>
__global__ void __launch_bounds__(64 * W, W == 4 ? 2 : 1) ring_attn_step_kernel(AttnArgs a) {
    constexpr int NT = 64 * W;          // threads
    constexpr int QT = 32 * W;          // queries per workgroup
    constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;          // 32-row blocks of O^T
    constexpr int KP = D + 8;           // K tile pitch (elements)
    // Transposed V tile pitch: 80 elements (160 bytes).  Measured on MI355X
    // (SQ_LDS_BANK_CONFLICT), pitches of 72 or 88 stall the LDS five times as
    // many cycles on bank conflicts as 80 or 112 (64-key tiles, d = 128).
    constexpr int VP = kKT + 16;
    constexpr int CH = kKT * D / 8;     // 16-byte chunks per K (or V) tile
    constexpr int CPT = CH / NT;        // chunks per thread
    static_assert(CH % NT == 0, "tile chunks must split evenly over the workgroup");
    // Two buffers of (K tile [key][d], V tile transposed [d][key]): the next
    // tile is staged into one while the other is read, one barrier a tile.
    extern __shared__ __attribute__((aligned(16))) __bf16 lds[];
    constexpr int KSZ = kKT * KP, BUF = kKT * KP + D * VP;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    // Workgroups go to the eight XCDs in turn (workgroup i to XCD i % 8), each
    // with its own L2.  Renumbered so that consecutive logical tiles, the
    // query tiles that stream the same K/V block, share an XCD and its L2.
    const uint32_t total = gridDim.x, lin = blockIdx.x;
    const uint32_t per = total / 8, rem = total % 8, xcd = lin % 8, slot = lin / 8;
    const uint32_t logical = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const uint32_t nq = (uint32_t)((a.s_local + QT - 1) / QT), nbh = (uint32_t)(a.b * a.heads);
    const uint32_t qtile = logical % nq, bh = (logical / nq) % nbh, sz = logical / nq / nbh;
    const int bi = (int)(bh / a.heads), hh = (int)(bh % a.heads);
    // Workgroup group sz covers ring steps first .. first + spg - 1, one after
    // another as one run of key tiles, and writes partial slot `part`.
    const int part = a.step0 + (int)sz, first = a.step0 + (int)sz * a.spg;
    const int64_t tok = a.b * a.heads * D;                     // elements per token
    const int64_t head_off = ((int64_t)bi * a.heads + hh) * D;
    const int64_t qrow = (int64_t)qtile * QT + wave * 32 + c;
    const int64_t qr = qrow < a.s_local ? qrow : a.s_local - 1;

    // Q^T operand: lane holds query c, d = 16*s + 8*g + 0..7.
    bf16x8 qv[KS];
    const __bf16* qp = a.q + qr * tok + head_off;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint4 w = load_stream(qp + 16 * s + 8 * g);
        qv[s] = __builtin_bit_cast(bf16x8, w);
    }

    // The run: for each ring step first .. first + spg - 1, the key tiles
    // k0 = 0, 64, ... of the block in hand at that step.  The fetch walks it one
    // tile ahead of the staging (f_k0, f_step: the next tile to fetch).
    const int64_t ntiles = (a.s_local + kKT - 1) / kKT * (RUN ? a.spg : 1);
    auto block_off = [&](int step) {
        const int blk = a.fused ? (a.rank - step % a.t + a.t) % a.t : 0;
        return (int64_t)blk * a.s_local * tok + head_off;
    };
    int64_t f_k0 = 0, f_boff = block_off(first);
    int f_step = first;

    // The next tile's K and V travel in registers while this tile is
    // computed.  K: chunk cc = tid + NT*i is key cc / (D/8), d = 8*(cc % (D/8)).
    // V: unit u = tid + NT*iu owns the 8-wide d chunk vdc = u % (D/8) of the R
    // columns R*q .. R*q+R-1, q = u / (D/8), which hold the consecutive keys
    // vpos(R*q) + 0..R-1; its transposed store is eight R-column runs (one
    // 2R-byte write each).
    constexpr int R = CPT >= 4 ? 4 : CPT;
    static_assert(CPT % R == 0 && (R == 1 || R == 2 || R == 4), "V is staged in runs of 1, 2 or 4 keys");
    uint4 kn[CPT], vn[CPT];
    // Per-thread byte offsets inside a tile (the tile's base is uniform).
    uint32_t koff[CPT], voff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int cc = tid + NT * i, key = cc / (D / 8), dc = cc % (D / 8);
        koff[i] = (uint32_t)(key * tok + 8 * dc) * 2u;
        const int u = tid + NT * (i / R), vdc = u % (D / 8), vkey = vpos(R * (u / (D / 8))) + (i % R);
        voff[i] = (uint32_t)(vkey * tok + 8 * vdc) * 2u;
    }
    auto fetch = [&]() {
        const int64_t k0 = f_k0;
        const __bf16* kb = a.k + f_boff;
        const __bf16* vb = a.v + f_boff;
        f_k0 += kKT;                                 // advance the run
        if constexpr (RUN) {
            if (f_k0 >= a.s_local) {                 // into the next step's block
                f_k0 = 0;
                f_boff = block_off(++f_step);
            }
        }
        const char* kt = reinterpret_cast<const char*>(kb + k0 * tok);
        const char* vt0 = reinterpret_cast<const char*>(vb + k0 * tok);
        if (k0 + kKT <= a.s_local) {                 // a whole tile (uniform)
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                kn[i] = load_stream(kt + koff[i]);
                vn[i] = load_stream(vt0 + voff[i]);
            }
        } else {                                     // the ragged last tile: clamp
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int cc = tid + NT * i, key = cc / (D / 8), dc = cc % (D / 8);
                const int64_t kk = k0 + key < a.s_local ? k0 + key : a.s_local - 1;
                kn[i] = load_stream(kb + kk * tok + 8 * dc);
                const int u = tid + NT * (i / R), vdc = u % (D / 8);
                const int vkey = vpos(R * (u / (D / 8))) + (i % R);
                const int64_t vk = k0 + vkey < a.s_local ? k0 + vkey : a.s_local - 1;
                vn[i] = load_stream(vb + vk * tok + 8 * vdc);
            }
        }
    };
    auto stage = [&](int buf) {
        __bf16* ks = lds + buf * BUF;
        __bf16* vt = ks + KSZ;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int cc = tid + NT * i, key = cc / (D / 8), dc = cc % (D / 8);
            *reinterpret_cast<uint4*>(&ks[key * KP + 8 * dc]) = kn[i];
        }
#pragma unroll
        for (int iu = 0; iu < CPT / R; ++iu) {
            const int u = tid + NT * iu, vdc = u % (D / 8), col = R * (u / (D / 8));
            bf16x8 v8[R];
#pragma unroll
            for (int j = 0; j < R; ++j) v8[j] = __builtin_bit_cast(bf16x8, vn[R * iu + j]);
            // rows 8*vdc + e share vswz (= 8*((vdc/2) % 8)): one column for all e
            __bf16* vrow = &vt[8 * vdc * VP + (col ^ vswz(8 * vdc))];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (R == 4) {
                    const bf16x4 run = {v8[0][e], v8[1][e], v8[2][e], v8[3][e]};
                    *reinterpret_cast<bf16x4*>(vrow + e * VP) = run;
                } else if constexpr (R == 2) {
                    const bf16x2 run = {v8[0][e], v8[1][e]};
                    *reinterpret_cast<bf16x2*>(vrow + e * VP) = run;
                } else {
                    vrow[e * VP] = v8[0][e];
                }
            }
        }
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = -INFINITY, l = 0.0f;      // running max (base-2 units) and sum of this query

    // Lane part of the V^T read column (see the O^T product below).
    const int vcol = 8 * (g ^ (c >> 4));
    fetch();
    stage(0);
    __syncthreads();
    if (ntiles > 1) fetch();
    int cur = 0;
    int64_t k0 = 0;                     // keys of the current tile within its block
    for (int64_t ti = 0; ti < ntiles; ++ti, k0 = (RUN && k0 + kKT >= a.s_local) ? 0 : k0 + kKT) {
        const __bf16* ks = lds + cur * BUF;
        const __bf16* vlane = ks + KSZ + c * VP;

        // S^T = K Q^T for keys 32*cb .. 32*cb+31 of the tile.
        // The two blocks' products alternate, so consecutive MFMAs are independent.
        f32x16 st[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) st[cb][r] = 0.0f;
        // Every K fragment is read before the first product (the reads
        // return in order, so each product waits for its own fragment only).
        bf16x8 kf[KS][2];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                kf[s][cb] = *reinterpret_cast<const bf16x8*>(&ks[(32 * cb + c) * KP + 16 * s + 8 * g]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) st[cb] = mfma32(kf[s][cb], qv[s], st[cb]);
        // Register r of block cb holds key 32*cb + 8*(r/4) + 4*g + r%4.  The
        // max is taken on the raw scores (the scale is positive) and the
        // scale enters through the exponent's FMA: p = 2^(s*c - m).
        if (k0 + kKT > a.s_local) {          // the last, ragged tile (uniform)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t key = k0 + 32 * cb + 8 * (r / 4) + 4 * g + (r % 4);
                    if (key >= a.s_local) st[cb][r] = -INFINITY;
                }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[cb][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        // The reference m moves only when a score exceeds it by more than
        // 2^kStale: the probabilities 2^(s*c - m) stay below 2^kStale (fine in
        // bf16 and in the fp32 sums), O / l and m + log2(l) do not depend on
        // which m is used, and the O rescale is skipped in nearly every tile.
        const float mt = tmax * a.scale_log2;                // finite: every tile has a key
        const float m_new = mt > m + kStale ? mt : m;
        float psum = 0.0f;
        bf16x8 pb[4];                               // P^T operands, keys as above
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p =
                    __builtin_amdgcn_exp2f(fmaf(st[kg >> 1][8 * (kg & 1) + e], a.scale_log2, -m_new));
                psum += p;
                pb[kg][e] = (__bf16)p;
            }
        psum += __shfl_xor(psum, 32);
        // Rescale O only when some query of the wave has a new maximum.
        if (__builtin_amdgcn_ballot_w64(m_new != m) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        l += psum;
        m = m_new;

        // O^T += V^T P^T.  Product kg covers keys kb + {4g..4g+3, 8+4g..8+4g+3},
        // kb = 32*(kg/2) + 16*(kg%2): the keys its P^T operand holds, columns
        // kb + 8g .. kb + 8g + 7 of row d = 32*db + c.  With vswz(d) =
        // 16*(db%4) + 8*(c/16) the column splits into a compile-time part in
        // bits 4-5, kb ^ 16*(db%4), and the lane part 8*(g ^ c/16) in bit 3.
        bf16x8 vf[4][DB];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int ct = (32 * (kg >> 1) + 16 * (kg & 1)) ^ (16 * (db & 3));
                vf[kg][db] = *reinterpret_cast<const bf16x8*>(vlane + 32 * db * VP + ct + vcol);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma32(vf[kg][db], pb[kg], o[db]);
        if (ti + 1 < ntiles) stage(cur ^ 1);   // the next tile, fetched a tile ago
        __syncthreads();            // staged tile visible; every wave is done with `cur`
        if (ti + 2 < ntiles) fetch();
        cur ^= 1;
    }

    // The partial of the workgroup's steps: O / l and its log-sum-exp
    // (natural log).
    if (qrow < a.s_local) {
        const int64_t row = ((int64_t)part * a.s_local + qrow) * a.b * a.heads +
                            (int64_t)bi * a.heads + hh;
        const float inv_l = 1.0f / l;
        float* po = a.part_o + row * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)   // d = 32*db + 8*q4 + 4*g + 0..3
                *reinterpret_cast<float4*>(po + 32 * db + 8 * q4 + 4 * g) =
                    make_float4(o[db][4 * q4] * inv_l, o[db][4 * q4 + 1] * inv_l,
                                o[db][4 * q4 + 2] * inv_l, o[db][4 * q4 + 3] * inv_l);
        if (g == 0) a.part_lse[row] = (m + __log2f(l)) * 0.69314718055994531f;
    }
}

// Merge: per (query, batch, head) row, the nparts partials in ring order.  A row
// is D/4 threads, each owning 4 consecutive d; the folded result is written
// as bf16 O and fp32 log-sum-exp.
template <int D>
__global__ void __launch_bounds__(256) ring_attn_merge_kernel(AttnArgs a) {
    constexpr int TPR = D / 4;
    const int64_t nrows = a.s_local * a.b * a.heads;
    const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int d0 = 4 * (threadIdx.x % TPR);
    if (row >= nrows) return;
    float lse = a.part_lse[row];
    float4 o = *reinterpret_cast<const float4*>(a.part_o + row * D + d0);
    for (int k = 1; k < a.nparts; ++k) {
        const int64_t pr = (int64_t)k * nrows + row;
        const float lk = a.part_lse[pr];
        const float4 ok = *reinterpret_cast<const float4*>(a.part_o + pr * D + d0);
        const float mx = fmaxf(lse, lk);
        const float wa = __expf(lse - mx), wb = __expf(lk - mx);
        const float inv = 1.0f / (wa + wb);
        o.x = (o.x * wa + ok.x * wb) * inv;
        o.y = (o.y * wa + ok.y * wb) * inv;
        o.z = (o.z * wa + ok.z * wb) * inv;
        o.w = (o.w * wa + ok.w * wb) * inv;
        lse = mx + __logf(wa + wb);
    }
    const uint32_t lo = pack_bf16x2(o.x, o.y), hi = pack_bf16x2(o.z, o.w);
    *reinterpret_cast<uint2*>(a.o_out + row * D + d0) = make_uint2(lo, hi);
    if (d0 == 0 && a.lse_out) a.lse_out[row] = lse;
}

template <int D, int W, bool RUN>
static hipError_t launch_step(const AttnArgs& a, int steps, hipStream_t s) {
    // One grid dimension: query tiles x (batch, head) x groups of steps, at
    // most 2^31 - 1 (the descriptor checks bound it).
    const dim3 g((unsigned)((a.s_local + 32 * W - 1) / (32 * W) * a.b * a.heads * steps));
    constexpr size_t lds = 2 * ((size_t)kKT * (D + 8) + (size_t)D * (kKT + 16)) * sizeof(__bf16);
    // The dynamic LDS allowance is set once per device (bit d of `done`).
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void*)ring_attn_step_kernel<D, W, RUN>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        done.fetch_or(bit, std::memory_order_release);
    }
    hipLaunchKernelGGL((ring_attn_step_kernel<D, W, RUN>), g, dim3(64 * W), lds, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_attn(const AttnArgs& a, int steps, bool step, bool merge, hipStream_t s) {
    // Eight waves: each staged tile serves 256 queries (the staging registers
    // and the L2 -> LDS traffic per query halve against four waves).
    if (step) {
        const hipError_t e = a.spg > 1 ? launch_step<D, kWaves, true>(a, steps, s)
                                       : launch_step<D, kWaves, false>(a, steps, s);
        if (e != hipSuccess) return e;
    }
    if (!merge) return hipSuccess;
    const int64_t nrows = a.s_local * a.b * a.heads;
    const int64_t rpb = 256 / (D / 4);
    hipLaunchKernelGGL(ring_attn_merge_kernel<D>, dim3((unsigned)((nrows + rpb - 1) / rpb)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

// steps: groups of ring steps in the step launch; step / merge: which of the
// two launches to make.
hipError_t launch_ring_attn(int d, const AttnArgs& a, int steps, bool step, bool merge,
                            hipStream_t s) {
    switch (d) {
        case 64: return launch_attn<64>(a, steps, step, merge, s);
        case 128: return launch_attn<128>(a, steps, step, merge, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spr

using namespace spr;

namespace {

bool attn_desc_ok(const spr_attn_desc* d) {
    if (!d) return false;
    if (d->s_local < 1 || d->b < 1 || d->heads < 1 || d->t < 1 || d->t > 65535) return false;
    if (d->rank < 0 || d->rank >= d->t) return false;
    if (d->d != 64 && d->d != 128) return false;
    if (d->b * (int64_t)d->heads > 65535) return false;
    if (!(d->scale >= 0.0f) || isinf(d->scale)) return false;               // also NaN
    if (d->steps_per_wg < 0 || d->steps_per_wg > d->t) return false;
    if (d->steps_per_wg > 0 && d->t % d->steps_per_wg != 0) return false;
    // every index (t blocks of s_local*b*heads*d elements) well inside 63 bits
    if ((double)d->t * (double)d->s_local * (double)d->b * d->heads * d->d > 4.0e18) return false;
    // all steps' query tiles in one launch dimension
    const int64_t qtiles = (d->s_local + 32 * kWaves - 1) / (32 * kWaves);
    if ((double)qtiles * (double)d->b * d->heads * d->t > 2147483647.0) return false;
    return true;
}

uint64_t rows_of(const spr_attn_desc* d) { return (uint64_t)d->s_local * d->b * d->heads; }

// Workspace: part_o (t*rows*d fp32), then part_lse (t*rows fp32), 256-aligned.
uint64_t part_o_bytes(const spr_attn_desc* d) {
    return ((uint64_t)d->t * rows_of(d) * d->d * 4u + 255u) & ~(uint64_t)255u;
}
uint64_t workspace_need(const spr_attn_desc* d) {
    return part_o_bytes(d) + (((uint64_t)d->t * rows_of(d) * 4u + 255u) & ~(uint64_t)255u);
}

// Ring steps per workgroup in the fused call: the largest divisor k of t
// that still leaves at least 256 workgroups (one per CU), so each workgroup
// walks a longer run of key tiles and the merge folds t / k partials instead
// of t (measured on MI355X, 4096 queries x 32768 keys, t = 8, the whole
// fused call: 4 steps per workgroup 549 us, 2: 565, 1: 600, 8 -- half the
// CUs idle -- 924).  desc.steps_per_wg = k asks for k (a divisor of t).
int steps_per_workgroup(const spr_attn_desc* d) {
    if (d->steps_per_wg > 0) return d->steps_per_wg;
    const int64_t per_step = (d->s_local + 32 * kWaves - 1) / (32 * kWaves) * d->b * d->heads;
    const int64_t cus = device_cu_count();
    int spg = 1;
    for (int k = 2; k <= d->t; ++k)
        if (d->t % k == 0 && per_step * (d->t / k) >= cus) spg = k;
    return spg;
}

AttnArgs make_args(const spr_attn_desc* d, void* workspace) {
    AttnArgs a{};
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_o_bytes(d));
    a.s_local = d->s_local;
    a.b = d->b;
    a.heads = d->heads;
    a.t = d->t;
    a.rank = d->rank;
    a.spg = 1;
    a.nparts = d->t;
    const double scale = d->scale > 0.0f ? (double)d->scale : 1.0 / sqrt((double)d->d);
    a.scale_log2 = (float)((double)(float)scale * 1.4426950408889634);
    return a;
}

}  // namespace

extern "C" {

size_t sp_ring_attn_workspace_bytes(const spr_attn_desc* d) {
    return attn_desc_ok(d) ? (size_t)workspace_need(d) : 0;
}

spr_status sp_ring_attn_step(const spr_attn_desc* d, int32_t step, const void* q,
                             const void* k_blk, const void* v_blk, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    if (!attn_desc_ok(d)) return SPR_ERR_INVALID_ARG;
    if (step < 0 || step >= d->t || !q || !k_blk || !v_blk) return SPR_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_blk, 16) || !aligned(v_blk, 16)) return SPR_ERR_INVALID_ARG;
    const uint64_t need = workspace_need(d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return SPR_ERR_WORKSPACE;
    const uint64_t blk = rows_of(d) * d->d * 2u;
    const Range outs[] = {range_of(workspace, need)};
    const Range ins[] = {range_of(q, blk), range_of(k_blk, blk), range_of(v_blk, blk)};
    if (!disjoint(outs, 1, ins, 3)) return SPR_ERR_INVALID_ARG;
    AttnArgs a = make_args(d, workspace);
    a.q = static_cast<const __bf16*>(q);
    a.k = static_cast<const __bf16*>(k_blk);
    a.v = static_cast<const __bf16*>(v_blk);
    a.step0 = step;
    a.fused = 0;
    return launch_ring_attn(d->d, a, 1, true, false, stream) == hipSuccess ? SPR_OK : SPR_ERR_HIP;
}

spr_status sp_ring_attn_merge(const spr_attn_desc* d, void* o_out, float* lse_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!attn_desc_ok(d) || !o_out) return SPR_ERR_INVALID_ARG;
    if (!aligned(o_out, 16) || !aligned(lse_out, 4)) return SPR_ERR_INVALID_ARG;
    const uint64_t need = workspace_need(d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return SPR_ERR_WORKSPACE;
    const Range outs[] = {range_of(o_out, rows_of(d) * d->d * 2u),
                          range_of(lse_out, rows_of(d) * 4u)};
    const Range ins[] = {range_of(workspace, need)};
    if (!disjoint(outs, 2, ins, 1)) return SPR_ERR_INVALID_ARG;
    AttnArgs a = make_args(d, workspace);
    a.o_out = static_cast<__bf16*>(o_out);
    a.lse_out = lse_out;
    return launch_ring_attn(d->d, a, 0, false, true, stream) == hipSuccess ? SPR_OK : SPR_ERR_HIP;
}

// Every check of the fused forward, then its launch arguments.
static spr_status prepare_fwd(const spr_attn_desc* d, const void* q, const void* k, const void* v,
                              void* o_out, float* lse_out, void* workspace,
                              size_t workspace_bytes, AttnArgs* out) {
    if (!attn_desc_ok(d)) return SPR_ERR_INVALID_ARG;
    if (!q || !k || !v || !o_out) return SPR_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_out, 16) ||
        !aligned(lse_out, 4))
        return SPR_ERR_INVALID_ARG;
    const uint64_t need = workspace_need(d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return SPR_ERR_WORKSPACE;
    const uint64_t blk = rows_of(d) * d->d * 2u;
    const Range outs[] = {range_of(o_out, blk), range_of(lse_out, rows_of(d) * 4u),
                          range_of(workspace, need)};
    const Range ins[] = {range_of(q, blk), range_of(k, blk * d->t), range_of(v, blk * d->t)};
    if (!disjoint(outs, 3, ins, 3)) return SPR_ERR_INVALID_ARG;
    AttnArgs a = make_args(d, workspace);
    a.q = static_cast<const __bf16*>(q);
    a.k = static_cast<const __bf16*>(k);
    a.v = static_cast<const __bf16*>(v);
    a.o_out = static_cast<__bf16*>(o_out);
    a.lse_out = lse_out;
    a.step0 = 0;
    a.fused = 1;
    a.spg = steps_per_workgroup(d);
    a.nparts = d->t / a.spg;
    *out = a;
    return SPR_OK;
}

spr_status sp_ring_attn_fwd(const spr_attn_desc* d, const void* q, const void* k,
                            const void* v, void* o_out, float* lse_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    AttnArgs a;
    const spr_status st = prepare_fwd(d, q, k, v, o_out, lse_out, workspace, workspace_bytes, &a);
    if (st != SPR_OK) return st;
    return launch_ring_attn(d->d, a, a.nparts, true, true, stream) == hipSuccess ? SPR_OK
                                                                                 : SPR_ERR_HIP;
}

int sp_ring_attn_fwd_num_launches(const spr_attn_desc* d) { return attn_desc_ok(d) ? 2 : 0; }

spr_status sp_ring_attn_fwd_launch(const spr_attn_desc* d, int index, const void* q, const void* k,
                                   const void* v, void* o_out, float* lse_out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    AttnArgs a;
    const spr_status st = prepare_fwd(d, q, k, v, o_out, lse_out, workspace, workspace_bytes, &a);
    if (st != SPR_OK) return st;
    if (index < 0 || index > 1) return SPR_ERR_INVALID_ARG;
    return launch_ring_attn(d->d, a, a.nparts, index == 0, index == 1, stream) == hipSuccess
               ? SPR_OK
               : SPR_ERR_HIP;
}

}  // extern "C"
