// sp_device.h -- device-side building blocks of the SP-region kernels (gfx950).
//
// Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC'11): written here for the GPU from
// the published round function; 32x32->64 products map to one v_mad_u64_u32.
// bf16 rounding uses the CDNA4 round-to-nearest-even convert
// (v_cvt_pk_bf16_f32).  Vectors are 16 bytes: 8 bf16 or 4 fp32 elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spr {

// ------------------------------------------------------------------ Philox
struct Philox4 {
    uint32_t w0, w1, w2, w3;
};

// Three-input XOR in one CDNA4 instruction (v_bitop3_b32, truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// One Philox4x32-10 block.  The key schedule adds the Weyl constants between
// rounds; c2/c3/k0/k1 are wave-uniform here, so the compiler keeps their
// first-round work on the scalar unit.  Per round: two 32x32->64 products
// (v_mad_u64_u32) and two three-input XORs.
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// Keep decisions of the 4 consecutive elements 4*blk .. 4*blk+3 of the full
// tensor: element 4*blk + j is kept iff word j >= thr.
__device__ __forceinline__ void keep4(uint64_t blk, uint32_t off_lo, uint32_t off_hi,
                                      uint32_t key_lo, uint32_t key_hi, uint32_t thr,
                                      bool* keep) {
    const Philox4 r = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), off_lo, off_hi,
                                    key_lo, key_hi);
    keep[0] = r.w0 >= thr;
    keep[1] = r.w1 >= thr;
    keep[2] = r.w2 >= thr;
    keep[3] = r.w3 >= thr;
}

// Mask word of 4 keep decisions: byte j is 1 when element j is kept.
// Keep decisions of the E consecutive elements from global element e0 (a
// multiple of 4) as bits: bit j set = element e0 + j kept.  The same words
// the forward drew (the backward regenerates them instead of reading a mask).
template <int E>
__device__ __forceinline__ uint32_t keep_bits(uint64_t e0, uint32_t off_lo, uint32_t off_hi,
                                              uint32_t key_lo, uint32_t key_hi, uint32_t thr) {
    uint32_t kb = 0;
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
        bool k4[4];
        keep4((e0 >> 2) + q, off_lo, off_hi, key_lo, key_hi, thr, k4);
#pragma unroll
        for (int j = 0; j < 4; ++j) kb |= (k4[j] ? 1u : 0u) << (4 * q + j);
    }
    return kb;
}

__device__ __forceinline__ uint32_t mask_word(const bool* keep) {
    return (keep[0] ? 1u : 0u) | (keep[1] ? 1u << 8 : 0u) | (keep[2] ? 1u << 16 : 0u) |
           (keep[3] ? 1u << 24 : 0u);
}

// ------------------------------------------------------------------ h
// residual + (keep ? (x + bias) * scale : 0), each operation a separately
// rounded fp32 operation: contraction into FMA is off for this body, so the
// result is bit-identical to the unfused sequence of IEEE operations.
__device__ __forceinline__ float residual_dropout(float x, float bias, float residual,
                                                  bool keep, float scale) {
#pragma clang fp contract(off)
    const float u = x + bias;
    const float v = keep ? u * scale : 0.0f;
    return residual + v;
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> one word of two bf16 (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------------ vectors
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte accesses: each byte of x, residual, h, y, dy, dx, dres is
// touched once per kernel, so they carry the nontemporal hint.
__device__ __forceinline__ uint4 load_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(void* p, uint4 q) {
    const u32x4_t v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// One 16-byte vector of the I/O type, widened to fp32.
template <typename IO> struct Vec;

template <> struct Vec<float> {
    static constexpr int N = 4;
    float v[4];
    __device__ __forceinline__ void set(uint4 q) {
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    }
    __device__ __forceinline__ uint4 get() const {
        return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                          __float_as_uint(v[3]));
    }
    __device__ __forceinline__ void load(const void* p) { set(load_stream(p)); }
    __device__ __forceinline__ void store(void* p) const { store_stream(p, get()); }
    // value as stored in the I/O type (identity for fp32)
    __device__ __forceinline__ static float round_io(float f) { return f; }
};

template <> struct Vec<__bf16> {
    static constexpr int N = 8;
    float v[8];
    __device__ __forceinline__ void set(uint4 q) {
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
        v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
        v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ __forceinline__ uint4 get() const {
        return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
    __device__ __forceinline__ void load(const void* p) { set(load_stream(p)); }
    __device__ __forceinline__ void store(void* p) const { store_stream(p, get()); }
    __device__ __forceinline__ static float round_io(float f) {
        return (float)(__bf16)f;
    }
};

// fp32 parameter slice matching one vector (4 or 8 floats, 16-byte aligned).
template <int N>
__device__ __forceinline__ void load_params(const float* p, float (&out)[N]) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
        const float4 q = *reinterpret_cast<const float4*>(p + i);
        out[i] = q.x; out[i + 1] = q.y; out[i + 2] = q.z; out[i + 3] = q.w;
    }
}

// Mask bytes of one vector (4 or 8 bytes; 1 = keep) from keep bits.
template <int N> struct MaskBytes;
template <> struct MaskBytes<4> {
    __device__ __forceinline__ static void store(uint8_t* p, uint32_t bits) {
        __builtin_nontemporal_store(
            (bits & 1u) | ((bits >> 1) & 1u) << 8 | ((bits >> 2) & 1u) << 16 | ((bits >> 3) & 1u) << 24,
            reinterpret_cast<uint32_t*>(p));
    }
    // any nonzero byte means keep
    __device__ __forceinline__ static uint32_t from_word(uint32_t w) {
        return (uint32_t)((w & 0xffu) != 0) | ((uint32_t)((w & 0xff00u) != 0) << 1) |
               ((uint32_t)((w & 0xff0000u) != 0) << 2) | ((uint32_t)((w & 0xff000000u) != 0) << 3);
    }
    __device__ __forceinline__ static uint32_t load(const uint8_t* p) {
        return from_word(*reinterpret_cast<const uint32_t*>(p));
    }
};
template <> struct MaskBytes<8> {
    __device__ __forceinline__ static void store(uint8_t* p, uint32_t bits) {
        const uint32_t lo = (bits & 1u) | ((bits >> 1) & 1u) << 8 | ((bits >> 2) & 1u) << 16 |
                            ((bits >> 3) & 1u) << 24;
        const uint32_t hi = ((bits >> 4) & 1u) | ((bits >> 5) & 1u) << 8 | ((bits >> 6) & 1u) << 16 |
                            ((bits >> 7) & 1u) << 24;
        __builtin_nontemporal_store(lo, reinterpret_cast<uint32_t*>(p));
        __builtin_nontemporal_store(hi, reinterpret_cast<uint32_t*>(p) + 1);
    }
    __device__ __forceinline__ static uint32_t load(const uint8_t* p) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        return MaskBytes<4>::from_word(w.x) | (MaskBytes<4>::from_word(w.y) << 4);
    }
};

// h of one vector: the stored words (for the h store) and the stored
// values widened back to fp32 (what the norm reads).
template <typename IO> struct HVec;
template <> struct HVec<__bf16> {
    __device__ __forceinline__ static void compute(uint4 xq, uint4 rq, const float (&b)[8],
                                                   const bool (&keep)[8], float scale,
                                                   uint4& hw, float (&hr)[8]) {
        const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w}, rw[4] = {rq.x, rq.y, rq.z, rq.w};
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float h0 = residual_dropout(bf16_lo(xw[p]), b[2 * p], bf16_lo(rw[p]),
                                              keep[2 * p], scale);
            const float h1 = residual_dropout(bf16_hi(xw[p]), b[2 * p + 1], bf16_hi(rw[p]),
                                              keep[2 * p + 1], scale);
            o[p] = pack_bf16x2(h0, h1);          // round to nearest even, two at a time
            hr[2 * p] = bf16_lo(o[p]);
            hr[2 * p + 1] = bf16_hi(o[p]);
        }
        hw = make_uint4(o[0], o[1], o[2], o[3]);
    }
};
template <> struct HVec<float> {
    __device__ __forceinline__ static void compute(uint4 xq, uint4 rq, const float (&b)[4],
                                                   const bool (&keep)[4], float scale,
                                                   uint4& hw, float (&hr)[4]) {
        const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w}, rw[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            hr[j] = residual_dropout(__uint_as_float(xw[j]), b[j], __uint_as_float(rw[j]),
                                     keep[j], scale);
        hw = make_uint4(__float_as_uint(hr[0]), __float_as_uint(hr[1]), __float_as_uint(hr[2]),
                        __float_as_uint(hr[3]));
    }
};

// ------------------------------------------------------------------ reductions
// Lane exchanges inside 16-lane rows by DPP (data-parallel primitives: the
// VALU reads the other lane's register directly, no LDS round trip).  Each
// control pairs a lane with one in the same row: quad_perm [1,0,3,2] and
// [2,3,0,1] swap neighbours at distance 1 and 2; row_half_mirror maps lane i
// of each 8-lane half to 7-i, row_mirror lane i of the row to 15-i.  Applied
// in that order to values that are already equal within the groups the
// earlier steps formed, each mirror pairs a group with its neighbour group,
// like an exchange at distance 4 and then 8.
enum : int {
    kDppXor1 = 0xB1,           // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,           // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141,    // row_half_mirror
    kDppMirror = 0x140         // row_mirror
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes of a wave, every lane getting the same bits: a
// butterfly inside each 16-lane row (each step adds the same two operands
// on both partners), then the four row sums, read from lanes 0, 16, 32 and
// 48, added as (r0 + r1) + (r2 + r3).  Needs all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Sum over the waves of a workgroup that owns one row.  `slot` points to
// 16 floats of LDS that no other live reduction uses; the partials are added
// in wave order, so every thread gets the same bits.
__device__ __forceinline__ float block_sum(float v, float* slot, int nwaves) {
    v = wave_sum(v);
    if (nwaves == 1) return v;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) slot[wave] = v;
    __syncthreads();
    float s = slot[0];
    for (int w = 1; w < nwaves; ++w) s += slot[w];
    return s;
}

// Running (count, mean, M2) of a set of values; merge() is Chan, Golub and
// LeVeque's pairwise update.  merge(a, b) is evaluated with `a` the operand
// from the lower lane (or earlier wave), so both butterfly partners compute
// the same expression and end with the same bits.
struct MeanM2 {
    float n, mean, m2;
};
__device__ __forceinline__ MeanM2 merge(MeanM2 a, MeanM2 b) {
    const float n = a.n + b.n;
    // b's weight nb / n through the hardware reciprocal: two instructions
    // instead of a correctly rounded division's ten, one rounding more;
    // both empty: (0, 0, 0)
    const float wb = n > 0.0f ? b.n * __builtin_amdgcn_rcpf(n) : 0.0f;
    const float d = b.mean - a.mean;
    return {n, a.mean + d * wb, a.m2 + b.m2 + d * d * a.n * wb};
}

// One butterfly step of the wave merge: partner by DPP control CTRL, the
// operand from the lower lane group first (bit `low` of the lane index
// clear), so both partners evaluate the same expression.
template <int CTRL>
__device__ __forceinline__ MeanM2 merge_step(MeanM2 v, int lane, int low) {
    const MeanM2 o{dpp<CTRL>(v.n), dpp<CTRL>(v.mean), dpp<CTRL>(v.m2)};
    const bool upper = (lane & low) != 0;
    return merge(upper ? o : v, upper ? v : o);
}

__device__ __forceinline__ MeanM2 lane_value(MeanM2 v, int lane) {
    return {lane_value(v.n, lane), lane_value(v.mean, lane), lane_value(v.m2, lane)};
}

// Team-wide merge of per-thread (count, mean, M2), the means taken relative
// to a pivot `piv` that is the same across each wave (a value of the row):
// DPP butterflies inside each wave's rows and its rows' results in row
// order, then the waves' results in wave order through `slot`
// (4 x 16 floats of LDS), each wave's mean first moved into wave 0's frame
// ((piv_w - piv_0) + mean_w, both differences of nearby values).  Returns
// the merge relative to wave 0's pivot, which `piv0` receives.  With the
// pivots the merged means stay of the size of the row's spread, not of its
// mean, so a row whose mean is many times its spread keeps its variance.
__device__ __forceinline__ MeanM2 block_mean_m2(MeanM2 v, float piv, float* slot, int nwaves,
                                                float& piv0) {
    const int lane = threadIdx.x & 63;
    v = merge_step<kDppXor1>(v, lane, 1);
    v = merge_step<kDppXor2>(v, lane, 2);
    v = merge_step<kDppHalfMirror>(v, lane, 4);
    v = merge_step<kDppMirror>(v, lane, 8);
    // the four rows' results, merged in row order
    v = merge(merge(lane_value(v, 0), lane_value(v, 16)),
              merge(lane_value(v, 32), lane_value(v, 48)));
    piv0 = piv;
    if (nwaves == 1) return v;
    const int wave = threadIdx.x >> 6;
    if (lane == 0) {
        slot[wave] = v.n; slot[16 + wave] = v.mean; slot[32 + wave] = v.m2; slot[48 + wave] = piv;
    }
    __syncthreads();
    piv0 = slot[48];
    MeanM2 acc{slot[0], slot[16], slot[32]};
    for (int w = 1; w < nwaves; ++w)
        acc = merge(acc, MeanM2{slot[w], (slot[48 + w] - piv0) + slot[16 + w], slot[32 + w]});
    return acc;
}

// Two sums at once (16 + 16 floats of LDS).
__device__ __forceinline__ void block_sum2(float& a, float& b, float* slot, int nwaves) {
    a = wave_sum(a);
    b = wave_sum(b);
    if (nwaves == 1) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { slot[wave] = a; slot[16 + wave] = b; }
    __syncthreads();
    float sa = slot[0], sb = slot[16];
    for (int w = 1; w < nwaves; ++w) { sa += slot[w]; sb += slot[16 + w]; }
    a = sa;
    b = sb;
}

}  // namespace spr
