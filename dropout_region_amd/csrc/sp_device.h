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

// One Philox4x32-10 block.  The key schedule adds the Weyl constants between
// rounds; c2/c3/k0/k1 are wave-uniform here, so the compiler keeps their
// first-round work on the scalar unit.
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// Keep bits of the 4 consecutive elements 4*blk .. 4*blk+3 of the full
// tensor: bit j set iff word j >= thr.
__device__ __forceinline__ uint32_t keep4(uint64_t blk, uint32_t off_lo, uint32_t off_hi,
                                         uint32_t key_lo, uint32_t key_hi, uint32_t thr) {
    const Philox4 r = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), off_lo, off_hi,
                                    key_lo, key_hi);
    return (uint32_t)(r.w0 >= thr) | ((uint32_t)(r.w1 >= thr) << 1) |
           ((uint32_t)(r.w2 >= thr) << 2) | ((uint32_t)(r.w3 >= thr) << 3);
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
// One 16-byte vector of the I/O type, widened to fp32.
template <typename IO> struct Vec;

template <> struct Vec<float> {
    static constexpr int N = 4;
    float v[4];
    __device__ __forceinline__ void load(const void* p) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ __forceinline__ void store(void* p) const {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
    // value as stored in the I/O type (identity for fp32)
    __device__ __forceinline__ static float round_io(float f) { return f; }
};

template <> struct Vec<__bf16> {
    static constexpr int N = 8;
    float v[8];
    __device__ __forceinline__ void load(const void* p) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
        v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
        v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ __forceinline__ void store(void* p) const {
        uint4 q;
        q.x = pack_bf16x2(v[0], v[1]);
        q.y = pack_bf16x2(v[2], v[3]);
        q.z = pack_bf16x2(v[4], v[5]);
        q.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(p) = q;
    }
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
        *reinterpret_cast<uint32_t*>(p) =
            (bits & 1u) | ((bits >> 1) & 1u) << 8 | ((bits >> 2) & 1u) << 16 | ((bits >> 3) & 1u) << 24;
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
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    }
    __device__ __forceinline__ static uint32_t load(const uint8_t* p) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        return MaskBytes<4>::from_word(w.x) | (MaskBytes<4>::from_word(w.y) << 4);
    }
};

// ------------------------------------------------------------------ reductions
// Sum over the 64 lanes of a wave; every lane gets the same bits (each
// butterfly step adds the same two operands on both partners).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
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
