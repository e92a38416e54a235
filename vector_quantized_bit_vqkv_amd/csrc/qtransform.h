// qtransform.h -- q' = H (q * s) for one query vector, by one wave, fp32.
//
// VecInfer summary card, "Summary": the queries get the inverse of the key
// transform (keys are divided by the per-channel smoothing scale s and rotated
// by a Hadamard matrix), so attention scores are unchanged.  With H the
// normalized Sylvester matrix (symmetric, H H = I), q' = H (q * s) gives
// q'.(H (k / s)) = q.k.
//
// Lane i holds elements 2i and 2i+1.  The first butterfly stage (h = 1) pairs
// those two in-lane; stage h >= 2 pairs lane i with lane i ^ (h / 2).  Six
// cross-lane stages, one multiply by 1/sqrt(128).  Every caller runs these
// same operations, so q' is bit-identical wherever it is computed.
#pragma once

#include "device_util.h"

namespace vqkv {

constexpr float kInvSqrtHeadDimF = 0x1.6a09e6p-4f;   // fp32 nearest to 1/sqrt(128)

// Lane's two query elements (raw: one word of two bf16, or two fp32 words)
// and their smoothing scales: the loads of the transform, kept apart so that
// a caller can issue them early and convert later.
struct QueryPair {
    uint32_t w0, w1;
    float s0, s1;
    int dtype;
};

// q points at the vector's first element, s at its KV head's smoothing scales.
__device__ __forceinline__ QueryPair load_query_pair(const void* q, int dtype, const float* s, int lane) {
    QueryPair r;
    r.dtype = dtype;
    if (dtype == 0) {
        // w1 is unused for bf16; it gets the neighbouring word of the row: a
        // constant or a copy of w0 would have to wait for a load in flight.
        r.w0 = *((const uint32_t*)q + lane);
        r.w1 = *((const uint32_t*)q + (lane ^ 1));
    } else {
        const uint2 w = *((const uint2*)q + lane);
        r.w0 = w.x;
        r.w1 = w.y;
    }
    r.s0 = s[2 * lane];
    r.s1 = s[2 * lane + 1];
    return r;
}

// The arithmetic of the transform; q_prime points at the output vector.  All
// 64 lanes of the wave must call it.
__device__ __forceinline__ void transform_query_pair(QueryPair v, float* q_prime, int lane) {
#pragma clang fp contract(off)                          // the same roundings whatever the file's flags
    // bf16: the two halves of w0 (exact); fp32: the two words.  Selects, not
    // branches, so the conversion stays here and not next to the loads.
    const bool bf = v.dtype == 0;
    const float x0_in = __builtin_bit_cast(float, bf ? (v.w0 << 16) : v.w0);
    const float x1_in = __builtin_bit_cast(float, bf ? (v.w0 & 0xffff0000u) : v.w1);
    float x0 = x0_in * v.s0;
    float x1 = x1_in * v.s1;
    // Stage h = 1.
    {
        const float a0 = x0, b0 = x1;
        x0 = a0 + b0;
        x1 = a0 - b0;
    }
    // Stages h = 2 .. 64: partner lane = lane ^ (h / 2); the lower index adds, the upper subtracts.
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(x0, m, 64);
        const float p1 = __shfl_xor(x1, m, 64);
        const bool upper = (lane & m) != 0;
        x0 = upper ? p0 - x0 : x0 + p0;
        x1 = upper ? p1 - x1 : x1 + p1;
    }
    float2 out;
    out.x = x0 * kInvSqrtHeadDimF;
    out.y = x1 * kInvSqrtHeadDimF;
    *((float2*)q_prime + lane) = out;
}

// q and q_prime point at the vector's first element; s at its KV head's
// smoothing scales.  All 64 lanes of the wave must call it.
__device__ __forceinline__ void transform_query_wave(const void* q, int dtype, const float* s, float* q_prime,
                                                     int lane) {
    transform_query_pair(load_query_pair(q, dtype, s, lane), q_prime, lane);
}

// Value-transform variant: out = s_v * (H o) for one fp32 output row o (the
// inverse of v' = H (v / s_v)), by one wave, with the butterflies above: lane
// i holds elements 2i and 2i+1, then one multiply by 1/sqrt(128) and one by
// s_v.  `in` and `out` may be the same row (every lane reads before it
// writes), in global memory or LDS.
__device__ __forceinline__ void value_untransform_wave(const float* in, const float* sv, float* out, int lane) {
#pragma clang fp contract(off)
    const float2 w = *((const float2*)in + lane);
    float x0 = w.x, x1 = w.y;
    {
        const float a0 = x0, b0 = x1;
        x0 = a0 + b0;
        x1 = a0 - b0;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(x0, m, 64);
        const float p1 = __shfl_xor(x1, m, 64);
        const bool upper = (lane & m) != 0;
        x0 = upper ? p0 - x0 : x0 + p0;
        x1 = upper ? p1 - x1 : x1 + p1;
    }
    float2 r;
    r.x = (x0 * kInvSqrtHeadDimF) * sv[2 * lane];
    r.y = (x1 * kInvSqrtHeadDimF) * sv[2 * lane + 1];
    *((float2*)out + lane) = r;
}

}  // namespace vqkv
