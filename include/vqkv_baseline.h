/*
 * vqkv_baseline.h -- measurement kernels shipped in libvqkv next to the VQ
 * path.  They are not part of the method; they give the numbers the VQ decode
 * is compared with.
 *
 * The VecInfer pages quote their attention speedups against an unquantized
 * FP16 KV cache ("VecInfer: ... Outlier-Suppressed Vector Quantization",
 * research.elamur.ai summary card, "Key points": up to 2.7x on H100 and 2.8x on
 * A100 for large-batch self-attention, Llama-3.1-8B, 196k tokens, 2-bit).
 * The same comparison on this GPU needs an unquantized decode written with
 * the same care; vqkv_baseline_bf16_decode is that kernel.
 * Conventions (pointers, streams, alignment, errors) as in vqkv.h.
 */
#ifndef VQKV_BASELINE_H
#define VQKV_BASELINE_H

#include <stddef.h>
#include <stdint.h>

#include "vqkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Split-context decode attention over a bf16 cache, same work split and
 * workspace format as vqkv_decode_attention (merge with vqkv_combine):
 * for each (b, g) and split, softmax(sm_scale * q.k) v over the split's tokens.
 *   shape      fmt is ignored; max_tokens is the bf16 cache capacity (multiple
 *              of 64); Hq / Hkv in {1, 2, 4, 5, 8}
 *   q          device, bf16 [B][Hq][128] (untransformed query)
 *   k, v       device, bf16 [B][Hkv][max_tokens][128]
 *   seq_len    host, 1 <= seq_len <= max_tokens
 *   num_splits host, 1 <= num_splits <= ceil(seq_len / 64)
 *   workspace  device, vqkv_workspace_bytes(shape, num_splits) bytes */
vqkv_status vqkv_baseline_bf16_decode(const vqkv_shape* shape, const void* q, const void* k, const void* v,
                                      int32_t seq_len, float sm_scale, int32_t num_splits, void* workspace,
                                      void* stream);

/* Reads `bytes` (rounded down to 16) of device memory once with 16-byte
 * loads: `blocks` work-groups of 1024 threads, each reading one contiguous
 * chunk; XOR-folds into sink[1024] (device) so the loads cannot be dropped.
 * Measures achievable HBM read bandwidth. */
vqkv_status vqkv_baseline_read_stream(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                                      void* stream);

/* vqkv_decode_attention on a kernel chosen for measurement instead of the
 * default one, so that the design choices stay measurable side by side:
 *   path 0  the default (the matrix-core kernel, every format)
 *   path 1  the score-lookup-table kernel (2-bit, Hq / Hkv <= 4): per
 *           work-group table of q'-by-centroid scores in LDS
 *   path 2  the gather kernel (2-bit and 1.5-bit): centroids gathered from
 *           the LDS codebooks, fp32 score products
 *   path 3  the matrix-core kernel, named explicitly
 * Same arguments, results (within the tolerance of each kernel's arithmetic)
 * and workspace format as vqkv_decode_attention; errors as in vqkv.h, with
 * the text from vqkv_last_error().  A path outside [0, 3] returns
 * VQKV_ERR_INVALID_ARG, a path that does not take the shape's format or
 * group size VQKV_ERR_UNSUPPORTED. */
vqkv_status vqkv_measure_decode_attention(const vqkv_shape* shape, const float* q_prime,
                                          const uint16_t* k_book, const uint16_t* v_book,
                                          const uint8_t* k_codes, const uint8_t* v_codes,
                                          int32_t seq_len, float sm_scale, int32_t num_splits,
                                          void* workspace, int32_t path, void* stream);

/* Message for the last failed baseline call on the calling thread. */
const char* vqkv_baseline_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VQKV_BASELINE_H */
