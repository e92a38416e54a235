// internal.h -- launch functions shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqkv {

// Byte offset of the value code of (token t, sub-vector j) in a 2-bit stream.
// Blocks of 64 tokens x 32 sub-vectors = 2048 bytes, cut into 64 chunks of 32
// bytes, chunk c being what lane c of the decode wave reads for the block:
// chunk 16*((j%16)/4) + 4*(t%4) + j%4, byte 2*((t%64)/4) + j/16.  In that
// order a lane's bytes are exactly the centroids it looks up for the value
// product, step by step (see the decode kernel).
__host__ __device__ __forceinline__ int64_t v_code_offset_2bit(int64_t t, int j) {
    const int u = (int)(t & 63);
    const int chunk = 16 * ((j & 15) >> 2) + 4 * (u & 3) + (j & 3);
    return (t >> 6) * 2048 + 32 * chunk + 2 * (u >> 2) + (j >> 4);
}

// Byte offset of the value code of (token t, sub-vector j), j < 64, in a 4-bit
// stream: blocks of 64 tokens x 64 sub-vectors = 4096 bytes, cut into 64
// chunks of 64 bytes; sub-vectors 2w and 2w + 1 sit where the 2-bit layout
// puts sub-vector w: chunk 16 ((w % 16) / 4) + 4 (u % 4) + w % 4 (u = t % 64),
// byte 4 (u / 4) + 2 (w / 16) + j % 2, i.e. the lane of a decode tile reads
// the codes of step s at dword s of its chunk.
__host__ __device__ __forceinline__ int64_t v_code_offset_4bit(int64_t t, int j) {
    const int u = (int)(t & 63), w = j >> 1;
    const int chunk = 16 * ((w & 15) >> 2) + 4 * (u & 3) + (w & 3);
    return (t >> 6) * 4096 + 64 * chunk + 4 * (u >> 2) + 2 * (w >> 4) + (j & 1);
}

// Byte offset of the 3-byte pair holding the value codes of sub-vectors
// (j, j + 8), j < 8, of token t in a 1.5-bit stream.  Blocks of 64 tokens x 16
// sub-vectors = 1536 bytes, cut into 32 streams of 48 bytes, stream
// 8*(j/2) + 2*(t%4) + j%2 holding the pair at bytes 3*((t%64)/4)..+2.  A stream
// is what lanes 2m and 2m+1 of the decode wave read for the block.
__host__ __device__ __forceinline__ int64_t v_pair_offset_1p5(int64_t t, int j) {
    const int u = (int)(t & 63);
    const int stream = 8 * (j >> 1) + 2 * (u & 3) + (j & 1);
    return (t >> 6) * 1536 + 48 * stream + 3 * (u >> 2);
}

// Byte offset of the 3-byte pair holding the value codes of sub-vectors
// (j, j + 16), j < 16, of token t in a 3-bit stream.  Blocks of 64 tokens x
// 32 sub-vectors = 3072 bytes, cut into 64 chunks of 48 bytes as in the 2-bit
// layout: chunk 16*(j/4) + 4*(t%4) + j%4 holds the pair at bytes
// 3*((t%64)/4)..+2.  Chunk c is what lane c of the decode wave reads.
__host__ __device__ __forceinline__ int64_t v_pair_offset_3bit(int64_t t, int j) {
    const int u = (int)(t & 63);
    const int chunk = 16 * ((j & 15) >> 2) + 4 * (u & 3) + (j & 3);
    return (t >> 6) * 3072 + 48 * chunk + 3 * (u >> 2);
}

// Bit position, from the start of a 1.25-bit value stream (b, h), of the
// 10-bit value code of (token t, sub-vector j), j < 16.  Blocks of 64 tokens x
// 16 sub-vectors = 1280 bytes, cut into 32 streams of 40 bytes in the 1.5-bit
// stream order: stream 8*((j%8)/2) + 2*(t%4) + j%2 holds the pairs (sub-vector
// j%8, sub-vector j%8 + 8) of its 16 tokens, pair (t%64)/4 in bits
// [20 ((t%64)/4), +20), sub-vector j in the pair's 10-bit half j / 8.  Two
// consecutive pairs (tokens u and u + 4 of one 8-token group) share five
// bytes: a writer of one token's pair keeps the other's bits.
__host__ __device__ __forceinline__ int64_t v_bit_1p25(int64_t t, int j) {
    const int u = (int)(t & 63);
    const int stream = 8 * ((j & 7) >> 1) + 2 * (u & 3) + (j & 1);
    return ((t >> 6) * 1280 + 40 * stream) * 8 + 20 * (u >> 2) + 10 * (j >> 3);
}

struct TransformQueryArgs {
    const void* q;          // [B][Hq][128], bf16 or fp32
    int dtype;              // 0 bf16, 1 fp32
    const float* smooth;    // [Hkv][128]
    float* q_prime;         // [B][Hq][128]
    int batch, hq, hkv;
};
hipError_t launch_transform_query(const TransformQueryArgs& a, hipStream_t stream);

struct AppendArgs {
    const void* k_new;      // [B][Hkv][n][128]
    const void* v_new;
    int dtype;
    int n_new, start_pos;
    const float* smooth;    // [Hkv][128]
    const uint16_t* k_book; // [Hkv][E][dsub]
    const uint16_t* v_book;
    uint8_t* k_codes;       // [B][Hkv][cap * W]
    uint8_t* v_codes;
    int batch, hkv, cap, fmt;
    const int32_t* positions;  // device [B] or null: one token per sequence at its own position
    const int32_t* block_table;  // device [B][Hkv][cap / 64] or null: codes in a pool of 64-token blocks
    int num_blocks;
    // Decode-step prologue (q_prime non-null): the key block of each (b, kv-head)
    // also writes q' = H (q * s) for the head's Hq / Hkv query heads (waves
    // 1..G, first) and clears the head's arrival counter for the decode.
    const void* q;          // [B][Hq][128], dtype as k_new
    float* q_prime;         // [B][Hq][128]
    int32_t* arrivals;      // [B][Hkv]
    int hq;
    int32_t* seq_lens_out;  // [B] or null: sequence b's length after the append, positions[b] + 1
                            // clamped to [0, cap] (with positions)
    const float* v_smooth;  // [Hkv][128] or null: value-transform variant, values coded as H (v / s_v)
};
hipError_t launch_quantize_append(const AppendArgs& a, hipStream_t stream);

struct DecodeArgs {
    const float* q_prime;   // [B][Hq][128]
    const uint16_t* k_book; // [Hkv][E][dsub]
    const uint16_t* v_book;
    const uint8_t* k_codes; // [B][Hkv][cap * W]
    const uint8_t* v_codes;
    float* part_o;          // [B][Hq][S][128]
    float* part_ml;         // [B][Hq][S][2]: (largest score, log2 of the split's weight sum), log2 units
    int batch, hq, hkv, cap, fmt;
    int seq_len, splits, chunk;
    float qscale;           // sm_scale * log2(e)
    int path;               // 0 auto, 1 score table (2-bit), 2 gather (2-bit, 1.5-bit), 3 matrix cores
    const int32_t* seq_lens;   // device [B] or null (then seq_len for every sequence)
    const int32_t* block_table;  // device [B][Hkv][cap / 64] or null: k_codes / v_codes are block pools
    int num_blocks;
    // Fused combine (matrix-core kernel only), out non-null: with one split the
    // work-group writes out directly; with more, each work-group counts itself
    // in arrivals[b][kv-head] (zero at launch) and the last one of a head
    // combines the head's splits into out and clears the counter.
    float* out;             // [B][Hq][128]
    int32_t* arrivals;      // [B][Hkv]
    const float* v_smooth;  // [Hkv][128] or null: with out, the output is mapped back, s_v * (H o)
    // Fused append (2-bit, one split, out non-null), app.k_new non-null: each
    // work-group first computes q' of its G query heads from app.q (q_prime is
    // not read) and codes the new token of its (b, kv-head) into app.k_codes /
    // app.v_codes, exactly as launch_quantize_append would; with app.positions,
    // sequence b's length is positions[b] + 1 clamped to [0, cap] (seq_lens
    // must be null).
    AppendArgs app;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

struct CombineArgs {
    const float* part_o;
    const float* part_ml;   // [B][Hq][S][2]
    float* out;             // [B][Hq][128]
    int batch, hq, splits;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// Value-transform variant: out[b][g] = s_v[h] * (H out[b][g]) in place.
struct ValueOutputArgs {
    float* out;             // [B][Hq][128]
    const float* v_smooth;  // [Hkv][128]
    int batch, hq, hkv;
};
hipError_t launch_value_output_transform(const ValueOutputArgs& a, hipStream_t stream);

// Workspace of the allocation-free decode step: a file-scope device array of
// kStaticScratchBytes (static_scratch.hip), one copy per GPU.  Returns the
// current device's copy's address (taken once per device with
// hipGetSymbolAddress, then kept) and, if `device` is not null, the device.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
hipError_t static_scratch(void** addr, int* device);

// Offline calibration.
hipError_t launch_smooth_scales(int hkv, int n_cal, const void* k_cal, int dtype, float* smooth,
                                hipStream_t stream);

struct TrainArgs {
    int fmt, n_cal, dtype, is_key, iters;
    const void* rows;       // [n_cal][128]
    const float* smooth;    // [128] (keys)
    const int64_t* init;    // [E] device
    uint16_t* book;         // [E][dsub] fp16 out
    double* centroids;      // [E][dsub] fp64 (workspace or caller buffer)
    double* points;         // [n_cal * 128] fp64 workspace
    int32_t* assign;        // [n_cal * J] workspace
};
hipError_t launch_train_codebook(const TrainArgs& a, hipStream_t stream);

}  // namespace vqkv
