// transform_query.hip -- q' = H (q * s) for every query head, fp32, in registers
// (the butterflies are in qtransform.h), and the value-transform variant's
// output map.  One wave per (b, g) vector.
#include "internal.h"
#include "qtransform.h"

namespace vqkv {

namespace {

__global__ __launch_bounds__(256) void transform_query_kernel(TransformQueryArgs a) {
    const int lane = threadIdx.x & 63;
    const int vec = blockIdx.x * 4 + (threadIdx.x >> 6);    // (b, g) flattened
    if (vec >= a.batch * a.hq) return;                      // whole wave leaves together
    const int g = vec % a.hq;
    const int h = g / (a.hq / a.hkv);
    const int64_t base = (int64_t)vec * kHeadDim;
    const size_t esz = a.dtype == 0 ? 2 : 4;
    transform_query_wave((const char*)a.q + base * esz, a.dtype, a.smooth + (int64_t)h * kHeadDim,
                         a.q_prime + base, lane);
}

// Value-transform variant: out[b][g] = s_v[h] * (H out[b][g]), in place, one
// wave per row.
__global__ __launch_bounds__(256) void value_output_transform_kernel(ValueOutputArgs a) {
    const int vec = blockIdx.x * 4 + (threadIdx.x >> 6);    // (b, g) flattened
    if (vec >= a.batch * a.hq) return;                      // whole wave leaves together
    const int h = (vec % a.hq) / (a.hq / a.hkv);
    float* row = a.out + (int64_t)vec * kHeadDim;
    value_untransform_wave(row, a.v_smooth + (int64_t)h * kHeadDim, row, threadIdx.x & 63);
}

}  // namespace

hipError_t launch_value_output_transform(const ValueOutputArgs& a, hipStream_t stream) {
    const int blocks = (a.batch * a.hq + 3) / 4;
    hipLaunchKernelGGL(value_output_transform_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_transform_query(const TransformQueryArgs& a, hipStream_t stream) {
    const int vecs = a.batch * a.hq;
    const int blocks = (vecs + 3) / 4;
    hipLaunchKernelGGL(transform_query_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vqkv
