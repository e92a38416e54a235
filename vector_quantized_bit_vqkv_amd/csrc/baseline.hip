// baseline.hip -- measurement kernels: a bf16 split-context decode attention
// over an unquantized KV cache (the comparison the VecInfer pages make: their
// speedups are quoted against an FP16 cache), and a plain HBM read stream that
// measures the bandwidth a streaming kernel reaches on this GPU.
//
// The bf16 decode uses the same grid, splits, online softmax and workspace
// format as vqkv_decode_attention, so vqkv_combine merges its splits.  Loads
// are fully coalesced: each wave instruction reads 1 KB = 4 consecutive tokens
// x 256 B; lane (r = lane / 16, c = lane % 16) holds dims [8c, 8c + 8) of
// token r of each 4-token block.  A token's score is reduced over its row of
// 16 lanes with DPP.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/vqkv.h"
#include "../../include/vqkv_baseline.h"
#include "attn_common.h"
#include "device_util.h"
#include "internal.h"

namespace vqkv {

namespace {

struct Bf16Args {
    const uint16_t* q;      // [B][Hq][128] bf16
    const uint16_t* k;      // [B][Hkv][cap][128] bf16
    const uint16_t* v;
};

__device__ __forceinline__ void unpack_bf16x8(const uint4 w, float (&f)[8]) {
    f[0] = bf16_bits_to_float(w.x & 0xffffu); f[1] = bf16_bits_to_float(w.x >> 16);
    f[2] = bf16_bits_to_float(w.y & 0xffffu); f[3] = bf16_bits_to_float(w.y >> 16);
    f[4] = bf16_bits_to_float(w.z & 0xffffu); f[5] = bf16_bits_to_float(w.z >> 16);
    f[6] = bf16_bits_to_float(w.w & 0xffffu); f[7] = bf16_bits_to_float(w.w >> 16);
}

template <int G, int NW>
__global__ __launch_bounds__(NW * 64) void bf16_decode_kernel(Bf16Args in, DecodeArgs a) {
    __shared__ __align__(16) float sbuf[NW][64 * G];
    __shared__ __align__(16) float merge[NW * G * (kHeadDim + 2)];
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane >> 4, c = lane & 15;
    const int t_begin = s * a.chunk;
    const int t_end = min(a.seq_len, t_begin + a.chunk);

    float qv[G][8];
    {
        const uint16_t* qp = in.q + ((int64_t)b * a.hq + h * G) * kHeadDim + 8 * c;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float f[8];
            unpack_bf16x8(*(const uint4*)(qp + g * kHeadDim), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) qv[g][i] = f[i] * a.qscale;
        }
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
    }
    const int64_t stream = (int64_t)b * a.hkv + h;
    const uint16_t* kbase = in.k + stream * (int64_t)a.cap * kHeadDim + 8 * c;
    const uint16_t* vbase = in.v + stream * (int64_t)a.cap * kHeadDim + 8 * c;
    float* sw = sbuf[wave];

    for (int tile = t_begin + wave * 64; tile < t_end; tile += NW * 64) {
#pragma unroll 4
        for (int blk = 0; blk < 16; ++blk) {
            const int t = tile + 4 * blk + r;
            float kf[8];
            unpack_bf16x8(*(const uint4*)(kbase + (int64_t)t * kHeadDim), kf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float part = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) part += qv[g][i] * kf[i];
                part = row_sum16(part);
                if (c == 0) sw[(4 * blk + r) * G + g] = t < t_end ? part : kNegInf;
            }
        }
        wave_lds_sync();
        float sc[G], p[G];
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = sw[lane * G + g];
        softmax_tile<G, 8>(sc, m, l, acc, p);
        wave_lds_sync();
#pragma unroll
        for (int g = 0; g < G; ++g) sw[lane * G + g] = p[g];
        wave_lds_sync();
#pragma unroll 4
        for (int blk = 0; blk < 16; ++blk) {
            const int t = tile + 4 * blk + r;
            float vf[8];
            unpack_bf16x8(*(const uint4*)(vbase + (int64_t)t * kHeadDim), vf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pv = sw[(4 * blk + r) * G + g];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[g][i] += pv * vf[i];
            }
        }
        wave_lds_sync();
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = wave_sum(l[g]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[g][i] += xor_lane(acc[g][i], 16);
            acc[g][i] += xor_lane(acc[g][i], 32);
        }
    }
    __syncthreads();
    merge_and_store<G, 8, NW>(merge, m, l, acc, a, b, h, s);
}

// Grid-stride read of `n16` 16-byte words; one xor per block keeps the loads live.
// Each block reads one contiguous chunk of the buffer, 1024 threads with four
// 16-byte loads in flight each (the pattern that reached the highest read rate
// in a sweep of grid-stride and chunked variants on MI355X).
__global__ __launch_bounds__(1024) void read_stream_kernel(const uint4* buf, int64_t n16, int64_t chunk,
                                                           uint32_t* sink) {
    uint32_t x = 0;
    const int64_t begin = (int64_t)blockIdx.x * chunk;
    const int64_t end = begin + chunk < n16 ? begin + chunk : n16;
    const int B = blockDim.x;
    int64_t i = begin + threadIdx.x;
    for (; i + 3 * B < end; i += 4 * B) {
        const uint4 a0 = buf[i], a1 = buf[i + B], a2 = buf[i + 2 * B], a3 = buf[i + 3 * B];
        x ^= a0.x ^ a0.y ^ a0.z ^ a0.w ^ a1.x ^ a1.y ^ a1.z ^ a1.w;
        x ^= a2.x ^ a2.y ^ a2.z ^ a2.w ^ a3.x ^ a3.y ^ a3.z ^ a3.w;
    }
    for (; i < end; i += B) {
        const uint4 a0 = buf[i];
        x ^= a0.x ^ a0.y ^ a0.z ^ a0.w;
    }
    // Store only on a value the data never folds to in practice; the compiler
    // still has to perform every load to decide.
    if (x == 0x9E3779B9u) sink[(blockIdx.x * blockDim.x + threadIdx.x) & 1023] = x;
}

thread_local char g_err[256] = "";

vqkv_status fail(vqkv_status st, const char* msg) {
    snprintf(g_err, sizeof(g_err), "%s", msg);
    return st;
}

}  // namespace
}  // namespace vqkv

extern "C" {

const char* vqkv_baseline_last_error(void) { return vqkv::g_err; }

vqkv_status vqkv_baseline_bf16_decode(const vqkv_shape* s, const void* q, const void* k, const void* v,
                                      int32_t seq_len, float sm_scale, int32_t num_splits, void* workspace,
                                      void* stream) {
    using namespace vqkv;
    if (!s || s->head_dim != 128 || s->batch < 1 || s->num_kv_heads < 1 || s->num_q_heads < 1 ||
        s->num_q_heads % s->num_kv_heads != 0 || s->max_tokens < 64 || s->max_tokens % 64 != 0)
        return fail(VQKV_ERR_INVALID_ARG, "bad shape");
    const int G = s->num_q_heads / s->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 5 && G != 8) return fail(VQKV_ERR_UNSUPPORTED, "group size");
    if (seq_len < 1 || seq_len > s->max_tokens) return fail(VQKV_ERR_INVALID_ARG, "seq_len");
    if (num_splits < 1 || num_splits > (seq_len + 63) / 64) return fail(VQKV_ERR_INVALID_ARG, "num_splits");
    if (!std::isfinite(sm_scale)) return fail(VQKV_ERR_INVALID_ARG, "sm_scale");
    if (!q || !k || !v || !workspace || (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)workspace) & 15))
        return fail(VQKV_ERR_INVALID_ARG, "pointer NULL or not 16-byte aligned");
    const size_t rows = (size_t)s->batch * s->num_q_heads * num_splits;
    const size_t o_bytes = (rows * 128 * sizeof(float) + 255) & ~(size_t)255;
    const int64_t tiles = (seq_len + 63) / 64;
    const int chunk = (int)(((tiles + num_splits - 1) / num_splits) * 64);
    DecodeArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, (float*)workspace,
                 (float*)((char*)workspace + o_bytes), s->batch, s->num_q_heads, s->num_kv_heads,
                 s->max_tokens, 0, seq_len, num_splits, chunk, (float)((double)sm_scale * 1.4426950408889634), 0};
    Bf16Args in{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v};
    const dim3 grid(num_splits, s->num_kv_heads, s->batch);
    constexpr int NW = 8;
    hipStream_t st = (hipStream_t)stream;
    switch (G) {
        case 1: hipLaunchKernelGGL((bf16_decode_kernel<1, NW>), grid, dim3(NW * 64), 0, st, in, a); break;
        case 2: hipLaunchKernelGGL((bf16_decode_kernel<2, NW>), grid, dim3(NW * 64), 0, st, in, a); break;
        case 4: hipLaunchKernelGGL((bf16_decode_kernel<4, NW>), grid, dim3(NW * 64), 0, st, in, a); break;
        case 5: hipLaunchKernelGGL((bf16_decode_kernel<5, NW>), grid, dim3(NW * 64), 0, st, in, a); break;
        case 8: hipLaunchKernelGGL((bf16_decode_kernel<8, NW>), grid, dim3(NW * 64), 0, st, in, a); break;
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? VQKV_OK : fail(VQKV_ERR_HIP, hipGetErrorString(e));
}

vqkv_status vqkv_baseline_read_stream(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
    using namespace vqkv;
    if (!buf || !sink || ((uintptr_t)buf & 15) || bytes < 16 || blocks < 1)
        return fail(VQKV_ERR_INVALID_ARG, "bad read-stream arguments");
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t chunk = (n16 + blocks - 1) / blocks;
    hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(1024), 0, (hipStream_t)stream, (const uint4*)buf,
                       n16, chunk, sink);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? VQKV_OK : fail(VQKV_ERR_HIP, hipGetErrorString(e));
}

}  // extern "C"
