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

// q and q_prime point at the vector's first element; s at its KV head's
// smoothing scales.  All 64 lanes of the wave must call it.
__device__ __forceinline__ void transform_query_wave(const void* q, int dtype, const float* s, float* q_prime,
                                                     int lane) {
#pragma clang fp contract(off)                          // the same roundings whatever the file's flags
    float x0, x1;
    if (dtype == 0) {
        const uint32_t w = *((const uint32_t*)q + lane);
        x0 = bf16_bits_to_float(w & 0xffffu);
        x1 = bf16_bits_to_float(w >> 16);
    } else {
        const float2 w = *((const float2*)q + lane);
        x0 = w.x;
        x1 = w.y;
    }
    x0 *= s[2 * lane];
    x1 *= s[2 * lane + 1];
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
