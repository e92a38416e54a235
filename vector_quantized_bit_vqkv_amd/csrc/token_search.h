// token_search.h -- the exact steps of coding one new key or value row,
// shared by the one-token append kernel and the decode kernel's fused append,
// so the two produce identical codes.
//
// VecInfer summary card, "Summary", and the arXiv 2510.06175 page's
// "technical framework" paragraph: a key is smoothed per channel (divided by
// s) and rotated by the normalized Hadamard transform; key and value
// sub-vectors are replaced by the index of their nearest codebook entry.  The
// fixed fp64 operation sequence (the same one the bulk kernels use):
//   x = k / s                     fp64 divide, correctly rounded
//   FWHT butterflies              stage h = 1, 2, ..., 64, pair (j, j + h) -> (a + b, a - b)
//   x *= 0x1.6a09e667f3bcdp-4     fp64 nearest 1/sqrt(128)
//   d_e = (x0 - c0)^2 + (x1 - c1)^2 + ...   left to right, no fused multiply-add
//   code = the lowest e with the smallest d_e
// Each function below turns contraction off inside its own body.
#pragma once

#include "device_util.h"

namespace vqkv {

constexpr double kInvSqrtHeadDimD = 0x1.6a09e667f3bcdp-4;

__device__ __forceinline__ double load_elem_d(const void* base, int64_t i, int dtype) {
    return (double)load_elem(base, i, dtype);
}

// Exact distance to a book entry already widened to fp64 (the same values
// as dist_h's conversions, so the same result), pinned order.
template <int DS>
__device__ __forceinline__ double dist_f64(const double* x, const double* c) {
#pragma clang fp contract(off)
    double t = x[0] - c[0];
    double d = t * t;
#pragma unroll
    for (int i = 1; i < DS; ++i) {
        t = x[i] - c[i];
        d = d + t * t;
    }
    return d;
}

// Exact distance to an fp16 book entry, pinned order.
template <int DS>
__device__ __forceinline__ double dist_h(const double* x, const uint16_t* c) {
#pragma clang fp contract(off)
    double t = x[0] - (double)half_bits_to_float(c[0]);
    double d = t * t;
#pragma unroll
    for (int i = 1; i < DS; ++i) {
        t = x[i] - (double)half_bits_to_float(c[i]);
        d = d + t * t;
    }
    return d;
}

// Lexicographic (distance, index) minimum over aligned groups of L lanes
// (L a power of two <= 64); every lane of a group gets its group's minimum.
template <int L>
__device__ __forceinline__ void group_argmin(double& d, int& idx) {
#pragma unroll
    for (int m = 1; m < L; m <<= 1) {
        const double od = __shfl_xor(d, m, 64);
        const int oi = __shfl_xor(idx, m, 64);
        if (od < d || (od == d && oi < idx)) { d = od; idx = oi; }
    }
}

// Normalized FWHT of one 128-value fp64 row in LDS by one wave (all 64 lanes
// call it): lane l holds x[l] and x[l + 64]; stage h < 64 exchanges between
// lanes l and l ^ h, stage 64 runs inside the lane.  The butterflies and their
// order are those listed above, so the result is bit-identical to a
// stage-by-stage FWHT over the row.
__device__ __forceinline__ void rotate_row_wave(double* x, int lane) {
#pragma clang fp contract(off)
    double lo = x[lane], hi = x[lane + 64];
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
        const double olo = __shfl_xor(lo, st, 64), ohi = __shfl_xor(hi, st, 64);
        if (lane & st) { lo = olo - lo; hi = ohi - hi; }
        else { lo = lo + olo; hi = hi + ohi; }
    }
    const double a0 = lo + hi, a1 = lo - hi;
    x[lane] = a0 * kInvSqrtHeadDimD;
    x[lane + 64] = a1 * kInvSqrtHeadDimD;
}

}  // namespace vqkv
