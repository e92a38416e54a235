// transform_query.hip -- q' = H (q * s) for every query head, fp32, in registers.
//
// VecInfer summary card, "Summary": the queries get the inverse of the key
// transform (keys are divided by the per-channel smoothing scale s and rotated
// by a Hadamard matrix), so attention scores are unchanged.  With H the
// normalized Sylvester matrix (symmetric, H H = I), q' = H (q * s) gives
// q'.(H (k / s)) = q.k.
//
// One wave per (b, g) vector.  Lane i holds elements 2i and 2i+1.  The first
// butterfly stage (h = 1) pairs those two in-lane; stage h >= 2 pairs lane i
// with lane i ^ (h / 2).  Six cross-lane stages, one multiply by 1/sqrt(128).
#include "device_util.h"
#include "internal.h"

namespace vqkv {

namespace {

constexpr float kInvSqrtHeadDim = 0x1.6a09e6p-4f;   // fp32 nearest to 1/sqrt(128)

__global__ __launch_bounds__(256) void transform_query_kernel(TransformQueryArgs a) {
    const int lane = threadIdx.x & 63;
    const int vec = blockIdx.x * 4 + (threadIdx.x >> 6);    // (b, g) flattened
    if (vec >= a.batch * a.hq) return;                      // whole wave leaves together
    const int g = vec % a.hq;
    const int h = g / (a.hq / a.hkv);
    const int64_t base = (int64_t)vec * kHeadDim + 2 * lane;
    const float* s = a.smooth + (int64_t)h * kHeadDim + 2 * lane;
    float x0, x1;
    if (a.dtype == 0) {
        const uint32_t w = *(const uint32_t*)((const uint16_t*)a.q + base);
        x0 = bf16_bits_to_float(w & 0xffffu);
        x1 = bf16_bits_to_float(w >> 16);
    } else {
        const float2 w = *(const float2*)((const float*)a.q + base);
        x0 = w.x;
        x1 = w.y;
    }
    x0 *= s[0];
    x1 *= s[1];
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
    out.x = x0 * kInvSqrtHeadDim;
    out.y = x1 * kInvSqrtHeadDim;
    *(float2*)(a.q_prime + base) = out;
}

}  // namespace

hipError_t launch_transform_query(const TransformQueryArgs& a, hipStream_t stream) {
    const int vecs = a.batch * a.hq;
    const int blocks = (vecs + 3) / 4;
    hipLaunchKernelGGL(transform_query_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vqkv
