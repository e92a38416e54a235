// device_util.h -- small device helpers shared by the libvqkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqkv {

constexpr int kHeadDim = 128;
constexpr int kWave = 64;

// ------------------------------------------------------------------ conversions

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Low and high fp16 halves of a dword, as floats (exact).
__device__ __forceinline__ float lo_half(uint32_t w) { return half_bits_to_float(w & 0xffffu); }
__device__ __forceinline__ float hi_half(uint32_t w) { return half_bits_to_float(w >> 16); }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// Element i of a row stored as bf16 (dtype 0) or fp32 (dtype 1); exact in fp32.
__device__ __forceinline__ float load_elem(const void* base, int64_t i, int dtype) {
    if (dtype == 0) return bf16_bits_to_float(((const uint16_t*)base)[i]);
    return ((const float*)base)[i];
}

// ----------------------------------------------------------- wave reductions
// DPP butterflies inside each row of 16 lanes, then the four row results are
// read out as scalars.  Every lane of the wave must be active.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float readlane(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));   // row_mirror
    return fmaxf(fmaxf(readlane(x, 0), readlane(x, 16)), fmaxf(readlane(x, 32), readlane(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
    x = x + dpp<0xB1>(x);
    x = x + dpp<0x4E>(x);
    x = x + dpp<0x141>(x);
    x = x + dpp<0x140>(x);
    return (readlane(x, 0) + readlane(x, 16)) + (readlane(x, 32) + readlane(x, 48));
}

// Sum over each row of 16 lanes; every lane of the row receives it.
__device__ __forceinline__ float row_sum16(float x) {
    x = x + dpp<0xB1>(x);
    x = x + dpp<0x4E>(x);
    x = x + dpp<0x141>(x);
    x = x + dpp<0x140>(x);
    return x;
}

// Value of x in lane (this lane ^ mask) for mask in {16, 32}.
__device__ __forceinline__ float xor_lane(float x, int mask) {
    return __shfl_xor(x, mask, kWave);
}

// Ordering point between a wave's own LDS writes and its later LDS reads of
// the same data.  A wavefront's LDS instructions execute in order, so the
// hardware needs no wait; this only stops the compiler from moving memory
// operations across it.  (A fence would also wait for every outstanding
// global load, including prefetches.)
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

}  // namespace vqkv
