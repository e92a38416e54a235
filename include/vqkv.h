/*
 * vqkv.h -- C ABI of libvqkv: decode self-attention that reads a
 * vector-quantized KV cache directly, for AMD Instinct MI355X (gfx950).
 *
 * The method is VecInfer's ("VecInfer: Efficient LLM Inference with Low-Bit KV
 * Cache via Outlier-Suppressed Vector Quantization"; summary card on
 * research.elamur.ai, sections "Summary" and "Key points"; arXiv 2510.06175
 * abstract and its "technical framework" paragraph):
 *   1. keys are smoothed per channel (divided by s) and rotated by a Hadamard
 *      transform; the query gets the matching inverse (times s, same rotation),
 *      so attention scores are unchanged;
 *   2. keys and values are stored as indices into K-Means codebooks:
 *      2^8 entries x 4 dims (2 bits per element) or 2^12 entries x 8 dims
 *      (1.5 bits per element);
 *   3. attention dequantizes inside the kernel, reading only the codes.
 *
 * Conventions for every call
 * --------------------------
 * - Pointers marked "device" point to GPU memory on the current HIP device;
 *   pointers marked "host" point to CPU memory.  The caller owns every buffer.
 *   The library never allocates, frees or synchronizes; all work is enqueued on
 *   `stream` (a hipStream_t; NULL means the null stream) and is asynchronous.
 * - Arguments are checked on the host before anything is enqueued.  A failed
 *   check returns VQKV_ERR_INVALID_ARG or VQKV_ERR_UNSUPPORTED and leaves device
 *   memory untouched.  A failed kernel launch returns VQKV_ERR_HIP.
 *   vqkv_last_error() then gives a message for the calling thread.
 * - head_dim is 128.  Hq must be a multiple of Hkv; q-head g uses KV head
 *   g / (Hq / Hkv).  G = Hq / Hkv must be in [1, 8].
 * - max_tokens (the cache capacity per (batch, KV head) stream) must be a
 *   positive multiple of 64.
 * - fp16 values are passed as their 16-bit patterns (uint16_t).
 * - Every device pointer must be aligned to 16 bytes.
 * - The library keeps no mutable global state; calls on different streams may
 *   run concurrently as long as they do not write the same buffers.
 *
 * Cache layout (per (batch, KV head) stream; streams are [B][Hkv] in that
 * order, each max_tokens * W bytes, W = vqkv_code_bytes_per_token(fmt)):
 * - Key codes, token-major: token t occupies bytes [t*W, (t+1)*W).  2-bit:
 *   byte j holds the code of sub-vector j (dims 4j..4j+3).  1.5-bit: the
 *   12-bit codes of sub-vectors 2i and 2i+1 (dims 8*2i.. and 8*(2i+1)..) share
 *   bytes 3i..3i+2 as b0 = c0 & 0xFF, b1 = (c0 >> 8) | ((c1 & 0xF) << 4),
 *   b2 = c1 >> 4.  3-bit: the same 12-bit pairs for sub-vectors 2i and 2i+1
 *   (dims 4*2i..), 48 bytes per token.  1.25-bit: 10-bit codes as
 *   little-endian bit fields (the same convention), sub-vector j in bits
 *   [10j, 10j + 10) of the token's 20 bytes.  4-bit: byte j holds the code of
 *   sub-vector j (dims 2j, 2j+1), 64 bytes per token.
 * - Value codes, blocked by tokens and arranged so that every lane of the
 *   decode kernel reads its codes for a block with one wide load.  2-bit:
 *   blocks of 64 tokens, 2048 bytes each, cut into 64 chunks of 32 bytes;
 *   the code of token t (u = t % 64) and sub-vector j sits in chunk
 *   16*((j%16)/4) + 4*(u%4) + j%4, at byte 2*(u/4) + j/16 of the chunk.
 *   1.5-bit: blocks of 64 tokens, 1536 bytes each, cut into 32 streams of 48
 *   bytes; the codes of sub-vectors j and j + 8 (j < 8) of token t form one
 *   12-bit pair (c0 = sub-vector j, packed by the rule above) in stream
 *   8*(j/2) + 2*(u%4) + j%2, bytes 3*(u/4)..3*(u/4)+2.  3-bit: blocks of 64
 *   tokens, 3072 bytes each, cut into 64 chunks of 48 bytes; the codes of
 *   sub-vectors j and j + 16 (j < 16) of token t form one 12-bit pair in chunk
 *   16*(j/4) + 4*(u%4) + j%4 (as in the 2-bit layout), bytes 3*(u/4)..+2.
 *   1.25-bit: blocks of 64 tokens, 1280 bytes each, cut into 32 streams of 40
 *   bytes in the 1.5-bit stream order (stream 8*(j/2) + 2*(u%4) + j%2 for the
 *   pair (j, j + 8), j < 8), the pair of token group u/4 in bits
 *   [20*(u/4), 20*(u/4) + 20) of the stream, sub-vector j in its low 10 bits.
 *   4-bit: blocks of 64 tokens, 4096 bytes each, cut into 64 chunks of 64
 *   bytes; sub-vectors 2w and 2w + 1 (4 dims) take the place of the 2-bit
 *   layout's sub-vector w: the code of token t and sub-vector j (w = j/2) sits
 *   in chunk 16*((w%16)/4) + 4*(u%4) + w%4, at byte 4*(u/4) + 2*(w/16) + j%2.
 * - Codebooks: fp16 [Hkv][E][dsub], one for keys and one for values per KV
 *   head, shared by every sub-vector position.  Key codebooks live in the
 *   rotated space.
 * - Smoothing scales: fp32 [Hkv][128], every entry finite and > 0 (not
 *   checked on device).
 */
#ifndef VQKV_H
#define VQKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VQKV_OK = 0,
    VQKV_ERR_INVALID_ARG = 1,   /* a null pointer, a bad size, misalignment, ... */
    VQKV_ERR_UNSUPPORTED = 2,   /* a well-formed request this build does not implement */
    VQKV_ERR_HIP = 3            /* the HIP runtime reported an error */
} vqkv_status;

typedef enum {
    VQKV_FMT_2BIT = 0,          /* 256 entries x 4 dims, uint8 codes, 32 B per token */
    VQKV_FMT_1P5BIT = 1,        /* 4096 entries x 8 dims, 12-bit codes, 24 B per token */
    /* A third width inside the pages' 1.25-4 bit range (the pages report that
     * range but print only the two shapes above): 4096 entries x 4 dims,
     * 12-bit codes, 3 bits per element, 48 B per token. */
    VQKV_FMT_3BIT = 2,
    /* The low end of that range: 1024 entries x 8 dims, 10-bit codes, 1.25 bits
     * per element, 20 B per token. */
    VQKV_FMT_1P25BIT = 3,
    /* The high end: 256 entries x 2 dims, uint8 codes, 4 bits per element,
     * 64 B per token. */
    VQKV_FMT_4BIT = 4,
    /* Flag OR'ed into any format: the value-transform variant.  The pages'
     * technical-framework paragraph quantizes the "preprocessed KV cache"; read
     * that way, values get their own per-channel scales s_v and the keys'
     * rotation, v' = H (v / s_v), are coded as v', and the attention output is
     * mapped back, o = s_v * (H o') (H is its own inverse).  Calls then take
     * smooth as [2][Hkv][128] (the keys' scales, then the values'). */
    VQKV_FMT_VALUE_TRANSFORM = 0x100
} vqkv_format;

typedef enum {
    VQKV_DTYPE_BF16 = 0,
    VQKV_DTYPE_FP32 = 1
} vqkv_dtype;

typedef struct {
    int32_t batch;              /* B >= 1 */
    int32_t num_q_heads;        /* Hq >= 1 */
    int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0, Hq / Hkv <= 8 */
    int32_t head_dim;           /* must be 128 */
    int32_t max_tokens;         /* cache capacity per stream, a positive multiple of 64 */
    int32_t fmt;                /* vqkv_format */
} vqkv_shape;

/* ------------------------------------------------------------- size queries */

/* Bytes per token per KV head for one of K or V: 32 (2-bit), 24 (1.5-bit),
 * 48 (3-bit), 20 (1.25-bit) or 64 (4-bit), with or without
 * VQKV_FMT_VALUE_TRANSFORM; 0 for an unknown format.  VecInfer card, "Key points" (codebook size). */
size_t vqkv_code_bytes_per_token(int32_t fmt);

/* Bytes of one code cache (keys or values): B * Hkv * max_tokens * W.
 * 0 if the shape is invalid. */
size_t vqkv_cache_bytes(const vqkv_shape* shape);

/* Bytes of the split-context workspace that vqkv_decode_attention writes and
 * vqkv_combine reads, for `num_splits` splits; 0 if the arguments are invalid. */
size_t vqkv_workspace_bytes(const vqkv_shape* shape, int32_t num_splits);

/* Bytes of the workspace of the vqkv_decode_step calls for `num_splits`
 * splits (the split partials, q', one counter per (b, KV head) and one length
 * per sequence); 0 if the arguments are invalid. */
size_t vqkv_step_workspace_bytes(const vqkv_shape* shape, int32_t num_splits);

/* A split count that fills the GPU for this shape and context length (>= 1):
 * about one work-group per compute unit of the current device (256 when no
 * device answers), at least 1024 tokens per split.  Any value in
 * [1, ceil(seq_len / 64)] is valid for the decode. */
int32_t vqkv_suggest_splits(const vqkv_shape* shape, int32_t seq_len);

/* Static text for a status code. */
const char* vqkv_status_string(int32_t status);

/* Message describing the last failed call on the calling thread ("" if none). */
const char* vqkv_last_error(void);

/* ---------------------------------------------------------- hot-path calls */

/* Query transform.  VecInfer card, "Summary": matching inverse operations on
 * the queries keep attention scores unchanged.  For each (b, g), with
 * h = g / G:  q'[b][g] = H (q[b][g] * s[h]), H the normalized 128 x 128
 * Sylvester Hadamard matrix, computed in fp32 by an in-register fast
 * Walsh-Hadamard transform.  Then q'.(H (k / s)) = q.k.
 *   q        device, [B][Hq][128], dtype q_dtype (vqkv_dtype)
 *   smooth   device, fp32 [Hkv][128] (with VQKV_FMT_VALUE_TRANSFORM its first
 *            half, the keys' scales)
 *   q_prime  device, fp32 [B][Hq][128] (output)
 * Only shape->batch, num_q_heads, num_kv_heads and head_dim are used. */
vqkv_status vqkv_transform_query(const vqkv_shape* shape, const void* q, int32_t q_dtype,
                                 const float* smooth, float* q_prime, void* stream);

/* Append quantizer.  VecInfer card, "Summary", and the arXiv page's three
 * stages (preprocess the keys, then vector-quantize the cache): for each new
 * token, x' = H (k / s_h) in fp64 (butterflies in stage order h = 1..64, then a
 * multiply by the fp64 nearest 1/sqrt(128)); for each sub-vector j the key
 * code is argmin_e sum_i (x'_{j*dsub+i} - C_K[e][i])^2, the value code the same
 * over the raw value and C_V, distances in fp64 summed left to right, ties to
 * the lowest index.  Codes are written for positions
 * [start_pos, start_pos + n_new) of every (b, h) stream; other positions keep
 * their bytes.
 *   k_new, v_new      device, [B][Hkv][n_new][128], dtype (vqkv_dtype)
 *   n_new             host, >= 1;  start_pos: host, >= 0,
 *                     start_pos + n_new <= max_tokens
 *   smooth            device, fp32 [Hkv][128]; [2][Hkv][128] with
 *                     VQKV_FMT_VALUE_TRANSFORM (the values are then coded as
 *                     H (v / s_v) with the same steps as the keys)
 *   k_book, v_book    device, fp16 [Hkv][E][dsub]
 *   k_codes, v_codes  device, cache buffers (layout above)
 * Calls that write the same stream must not overlap in time. */
vqkv_status vqkv_quantize_append(const vqkv_shape* shape, const void* k_new, const void* v_new,
                                 int32_t dtype, int32_t n_new, int32_t start_pos,
                                 const float* smooth, const uint16_t* k_book,
                                 const uint16_t* v_book, uint8_t* k_codes, uint8_t* v_codes,
                                 void* stream);

/* Ragged batches: one new token per sequence, sequence b's at position
 * positions[b] (the codes it computes are those of vqkv_quantize_append).
 *   k_new, v_new  device, [B][Hkv][1][128], dtype
 *   positions     device, int32 [B], 4-byte aligned; a position outside
 *                 [0, max_tokens) leaves that sequence's cache untouched
 *   other arguments as for vqkv_quantize_append. */
vqkv_status vqkv_quantize_append_varlen(const vqkv_shape* shape, const void* k_new, const void* v_new,
                                        int32_t dtype, const int32_t* positions, const float* smooth,
                                        const uint16_t* k_book, const uint16_t* v_book, uint8_t* k_codes,
                                        uint8_t* v_codes, void* stream);

/* Split-context decode attention over the codes.  VecInfer abstract: a kernel
 * that fuses dequantization into the attention computation to minimize memory
 * access.  For each (b, g) and split i of `num_splits` equal 64-aligned token
 * ranges of [0, seq_len):
 *   z_t = sm_scale * q'[b][g] . concat_j C_K[kc_t,j];
 *   o_i = sum_t softmax_i(z)_t * concat_j C_V[vc_t,j],  lse_i = log-sum-exp of z
 * over the split's tokens (online softmax), written to `workspace`.
 *   q_prime           device, fp32 [B][Hq][128] (from vqkv_transform_query)
 *   k_book, v_book    device, fp16 [Hkv][E][dsub]
 *   k_codes, v_codes  device, cache buffers holding tokens [0, seq_len)
 *   seq_len           host, 1 <= seq_len <= max_tokens
 *   sm_scale          host, finite (usually 1/sqrt(128))
 *   num_splits        host, 1 <= num_splits <= ceil(seq_len / 64)
 *   workspace         device, vqkv_workspace_bytes(shape, num_splits) bytes;
 *                     its contents are private to vqkv_combine. */
vqkv_status vqkv_decode_attention(const vqkv_shape* shape, const float* q_prime,
                                  const uint16_t* k_book, const uint16_t* v_book,
                                  const uint8_t* k_codes, const uint8_t* v_codes,
                                  int32_t seq_len, float sm_scale, int32_t num_splits,
                                  void* workspace, void* stream);

/* Ragged batches: sequence b holds seq_lens[b] tokens.  The same computation
 * as vqkv_decode_attention per sequence; every sequence is cut into the same
 * num_splits ranges of ceil(max_seq_len / num_splits) tokens (64-aligned), so
 * splits past a short sequence's end are empty (their lse is -inf and
 * vqkv_combine skips them).  A sequence of length 0 gets a zero output.
 *   seq_lens      device, int32 [B], 4-byte aligned; each value is clamped on
 *                 the device to [0, max_tokens], so no value can make the
 *                 kernel read outside the cache (values above max_seq_len are
 *                 an error the caller must avoid: tokens past the last split
 *                 would be ignored)
 *   max_seq_len   host, 1 <= max_seq_len <= max_tokens, >= every seq_lens[b]
 *   num_splits    host, 1 <= num_splits <= ceil(max_seq_len / 64)
 *   other arguments as for vqkv_decode_attention. */
vqkv_status vqkv_decode_attention_varlen(const vqkv_shape* shape, const float* q_prime,
                                         const uint16_t* k_book, const uint16_t* v_book,
                                         const uint8_t* k_codes, const uint8_t* v_codes,
                                         const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                         int32_t num_splits, void* workspace, void* stream);

/* Paged caches: the codes of each (b, KV head) stream live in 64-token blocks
 * of a shared pool, block_table naming the pool block of each logical block
 * (the 64-token blocks of the cache layout above, each 64 * W bytes).  Same
 * computation and arguments as vqkv_decode_attention_varlen, with
 *   k_pool, v_pool  device, [num_blocks][64 * W] bytes each
 *   num_blocks      host, >= 1
 *   block_table     device, int32 [B][Hkv][max_tokens / 64], 4-byte aligned;
 *                   entries are clamped to [0, num_blocks) on the device
 * Runs on the matrix-core kernel only (a measurement override to another
 * kernel returns VQKV_ERR_UNSUPPORTED). */
vqkv_status vqkv_decode_attention_paged(const vqkv_shape* shape, const float* q_prime,
                                        const uint16_t* k_book, const uint16_t* v_book,
                                        const uint8_t* k_pool, const uint8_t* v_pool, int32_t num_blocks,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        int32_t max_seq_len, float sm_scale, int32_t num_splits,
                                        void* workspace, void* stream);

/* Paged caches: one new token per sequence at positions[b] (as
 * vqkv_quantize_append_varlen), written into the pool block the table names
 * for its logical block.  Pool and table as for vqkv_decode_attention_paged. */
vqkv_status vqkv_quantize_append_paged(const vqkv_shape* shape, const void* k_new, const void* v_new,
                                       int32_t dtype, const int32_t* positions, const float* smooth,
                                       const uint16_t* k_book, const uint16_t* v_book, uint8_t* k_pool,
                                       uint8_t* v_pool, int32_t num_blocks, const int32_t* block_table,
                                       void* stream);

/* Log-sum-exp merge of the splits.  VecInfer card, "Summary": the attention
 * kernel tiles the context; its "References" name the decoding scheme this
 * finishes, a context cut into independent splits whose partial softmax
 * results are merged afterwards (FlashDecoding++, reference 15), with the
 * online normalizer of reference 26.  Split i contributes (o_i, lse_i), its
 * normalized output and the log-sum-exp of its scores:
 * out[b][g] = sum_i exp(lse_i - L) o_i, L = log sum_i exp(lse_i); a split
 * with no token (lse_i = -inf) weighs 0, and a row with no token gives 0.
 * The workspace holds each lse_i as two numbers, the split's largest score
 * and the log of its weight sum, so the weights keep full fp32 precision
 * whatever the size of the scores.
 *   workspace   device, as written by vqkv_decode_attention with the same
 *               shape and num_splits
 *   out         device, fp32 [B][Hq][128] (output; with VQKV_FMT_VALUE_TRANSFORM
 *               still in the rotated value space: vqkv_value_output_transform
 *               maps it back) */
vqkv_status vqkv_combine(const vqkv_shape* shape, int32_t num_splits, const void* workspace,
                         float* out, void* stream);

/* One decode step: the append of one new token per sequence at `position`,
 * the query transform, the attention of every query over tokens
 * [0, position] and the split combine.  The result is bit-identical to the
 * four calls
 *   vqkv_quantize_append(n_new = 1, start_pos = position), vqkv_transform_query,
 *   vqkv_decode_attention(seq_len = position + 1), vqkv_combine
 * on the same arguments (the same kernels' arithmetic).  Runs on the
 * matrix-core kernel, in one to three launches:
 *   - 2-bit without VQKV_FMT_VALUE_TRANSFORM: the attention kernel appends
 *     the token (in the work-group whose split holds `position`) and
 *     transforms its queries itself; with one split it writes `out` directly
 *     (one launch), with more it writes the splits' partials to the
 *     workspace and vqkv_combine's kernel merges them (two launches);
 *   - the other formats: an append launch that also transforms the query,
 *     then the attention: with one split it writes `out` directly (two
 *     launches), with more it writes the splits' partials and vqkv_combine's
 *     kernel merges them (three launches);
 *   - with VQKV_FMT_VALUE_TRANSFORM and more than one split: the append
 *     launch, then the attention, where the last split of each (b, KV head)
 *     to finish combines that head's splits and maps the output back (a
 *     per-head arrival counter in the workspace, cleared by the append launch
 *     of every step, so the workspace needs no initialization).
 *   q                 device, [B][Hq][128], dtype (the same dtype as k_new)
 *   k_new, v_new      device, [B][Hkv][1][128], dtype
 *   position          host, 0 <= position < max_tokens
 *   num_splits        host, 1 <= num_splits <= ceil((position + 1) / 64)
 *   workspace         device, vqkv_step_workspace_bytes(shape, num_splits)
 *                     bytes, private to the call; steps sharing a workspace
 *                     must not overlap in time
 *   out               device, fp32 [B][Hq][128] (output; with
 *                     VQKV_FMT_VALUE_TRANSFORM already mapped back, as
 *                     vqkv_value_output_transform would)
 *   other arguments as for vqkv_quantize_append and vqkv_decode_attention. */
vqkv_status vqkv_decode_step(const vqkv_shape* shape, const void* q, const void* k_new, const void* v_new,
                             int32_t dtype, int32_t position, const float* smooth, const uint16_t* k_book,
                             const uint16_t* v_book, uint8_t* k_codes, uint8_t* v_codes, float sm_scale,
                             int32_t num_splits, void* workspace, float* out, void* stream);

/* Bytes of the static scratch behind vqkv_decode_step_static, on each GPU. */
#define VQKV_STATIC_SCRATCH_BYTES ((size_t)8 << 20)

/* vqkv_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same computation, kernels and result bits as vqkv_decode_step (same
 * arguments, checks and errors, minus `workspace`); the step's workspace is
 * a static device array of VQKV_STATIC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends.  Neither the call nor the
 * library allocates or frees memory.
 * - A shape and split count whose vqkv_step_workspace_bytes exceeds
 *   VQKV_STATIC_SCRATCH_BYTES return VQKV_ERR_UNSUPPORTED, with no device work
 *   (for example batch 32 x 32 query heads fits up to 14 splits).
 * - Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents; the step needs none of them (its arrival counters are
 *   cleared by its own append launch, as with a caller's workspace).
 * - Calls that overlap in time on one GPU (other streams, other threads)
 *   race on the array: the caller must serialize them. */
vqkv_status vqkv_decode_step_static(const vqkv_shape* shape, const void* q, const void* k_new,
                                    const void* v_new, int32_t dtype, int32_t position, const float* smooth,
                                    const uint16_t* k_book, const uint16_t* v_book, uint8_t* k_codes,
                                    uint8_t* v_codes, float sm_scale, int32_t num_splits, float* out,
                                    void* stream);

/* The fused step for ragged batches: sequence b's new token lands at
 * positions[b] and its queries attend to tokens [0, positions[b]].  The result
 * is bit-identical to vqkv_quantize_append_varlen(positions),
 * vqkv_transform_query, vqkv_decode_attention_varlen(seq_lens = positions + 1,
 * max_seq_len) and vqkv_combine; a position outside [0, max_tokens) leaves the
 * cache untouched and its length is clamped to [0, max_tokens] as in the
 * varlen decode (a negative position gives a zero output).  The lengths are
 * derived from positions on the device (into the workspace when an append
 * launch runs first).
 *   positions     device, int32 [B], 4-byte aligned
 *   max_seq_len   host, 1 <= max_seq_len <= max_tokens, >= every positions[b] + 1
 *                 (a position past the last split's tokens is still appended,
 *                 but no split attends to it, as with the separate calls)
 *   num_splits    host, 1 <= num_splits <= ceil(max_seq_len / 64)
 *   other arguments as for vqkv_decode_step. */
vqkv_status vqkv_decode_step_varlen(const vqkv_shape* shape, const void* q, const void* k_new,
                                    const void* v_new, int32_t dtype, const int32_t* positions,
                                    int32_t max_seq_len, const float* smooth, const uint16_t* k_book,
                                    const uint16_t* v_book, uint8_t* k_codes, uint8_t* v_codes,
                                    float sm_scale, int32_t num_splits, void* workspace, float* out,
                                    void* stream);

/* The fused step for paged caches: as vqkv_decode_step_varlen, with the codes
 * in a pool of 64-token blocks named by block_table (pool and table as for
 * vqkv_decode_attention_paged); bit-identical to vqkv_quantize_append_paged,
 * vqkv_transform_query, vqkv_decode_attention_paged and vqkv_combine,
 * provided that the pool block receiving a sequence's new token is named by no
 * other table entry the step reads (another logical block below some
 * sequence's length): for 2-bit the append and the attention share one launch,
 * so a work-group reading such a block may see it before or after the write. */
vqkv_status vqkv_decode_step_paged(const vqkv_shape* shape, const void* q, const void* k_new,
                                   const void* v_new, int32_t dtype, const int32_t* positions,
                                   int32_t max_seq_len, const float* smooth, const uint16_t* k_book,
                                   const uint16_t* v_book, uint8_t* k_pool, uint8_t* v_pool,
                                   int32_t num_blocks, const int32_t* block_table, float sm_scale,
                                   int32_t num_splits, void* workspace, float* out, void* stream);

/* Value-transform variant (shape->fmt has VQKV_FMT_VALUE_TRANSFORM): maps
 * attention outputs of the rotated values back, in place:
 * out[b][g] = s_v[h] * (H out[b][g]), h = g / G, with the same fp32
 * butterflies as vqkv_transform_query, then a multiply by the fp32 nearest
 * 1/sqrt(128) and one by s_v.  Apply it to the output of vqkv_combine; the
 * vqkv_decode_step calls apply it themselves.
 *   smooth   device, fp32 [2][Hkv][128] (keys' scales, then values')
 *   out      device, fp32 [B][Hq][128], in place
 * A shape without the flag returns VQKV_ERR_INVALID_ARG. */
vqkv_status vqkv_value_output_transform(const vqkv_shape* shape, const float* smooth, float* out,
                                        void* stream);

/* ------------------------------------------------- offline calibration calls */

/* Smoothing scales.  VecInfer card, "Summary" (channel-wise smoothing of the
 * keys); the scale is not printed on the pages: this library uses
 * s[h][c] = sqrt(max_t |k_cal[h][t][c]|), the fp32 nearest the fp64 root.
 *   k_cal    device, [Hkv][n_cal][128], dtype;  n_cal >= 1 (host)
 *   smooth   device, fp32 [Hkv][128] (output) */
vqkv_status vqkv_smooth_scales(int32_t num_kv_heads, int32_t n_cal, const void* k_cal,
                               int32_t dtype, float* smooth, void* stream);

/* Bytes of device workspace vqkv_train_codebook needs for n_cal tokens. */
size_t vqkv_train_workspace_bytes(int32_t fmt, int32_t n_cal);

/* Offline K-Means codebook for one KV head (VecInfer card, "Summary": a
 * K-Means codebook trained offline).  The points are the sub-vectors of the
 * n_cal calibration rows: for keys (is_key != 0) the rotated x' = H (k / s),
 * for values the raw rows.  Lloyd iterations from the initial points
 * `init_idx` (device int64 [E], distinct indices into the n_cal * (128 / dsub)
 * points, point p = row p / J, sub-vector p % J; an index outside that range
 * is clamped into it): assign each point to its nearest
 * centroid (same fp64 rule as vqkv_quantize_append), then move each centroid
 * to the mean of its points; a centroid without points stays.  After `iters`
 * iterations the centroids are rounded to fp16 (nearest, ties to even).
 *   rows       device, [n_cal][128], dtype
 *   smooth     device, fp32 [128] (keys only; may be NULL for values)
 *   book       device, fp16 [E][dsub] (output)
 *   centroids  device, fp64 [E][dsub] (output, before rounding; may be NULL)
 *   workspace  device, vqkv_train_workspace_bytes(fmt, n_cal) bytes
 * Each centroid's sum is accumulated in fp64 in increasing point order, so the
 * result does not depend on scheduling and is the same on every run. */
vqkv_status vqkv_train_codebook(int32_t fmt, int32_t n_cal, const void* rows, int32_t dtype,
                                int32_t is_key, const float* smooth, const int64_t* init_idx,
                                int32_t iters, uint16_t* book, double* centroids,
                                void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQKV_H */
