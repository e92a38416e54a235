// capi.cpp -- the extern "C" boundary of libvqkv: argument checks on the host,
// then kernel launches on the caller's stream.  No allocation, no
// synchronization, no global mutable state besides the per-thread error text.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "../../include/vqkv.h"
#include "../../include/vqkv_baseline.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

vqkv_status fail(vqkv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

vqkv_status ok() {
    g_last_error[0] = '\0';
    return VQKV_OK;
}

vqkv_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(VQKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The code format without the variant flag, and the values' scales of the
// value-transform variant (the second half of smooth) or null.
int base_fmt(int fmt) { return fmt & 0xff; }
const float* value_scales(const vqkv_shape* s, const float* smooth) {
    return (s->fmt & VQKV_FMT_VALUE_TRANSFORM) ? smooth + (int64_t)s->num_kv_heads * 128 : nullptr;
}

int entries_of(int fmt) {
    return (fmt == VQKV_FMT_2BIT || fmt == VQKV_FMT_4BIT) ? 256 : (fmt == VQKV_FMT_1P25BIT ? 1024 : 4096);
}
int dsub_of(int fmt) {
    return (fmt == VQKV_FMT_1P5BIT || fmt == VQKV_FMT_1P25BIT) ? 8 : (fmt == VQKV_FMT_4BIT ? 2 : 4);
}
bool known_fmt(int fmt) {
    return fmt == VQKV_FMT_2BIT || fmt == VQKV_FMT_1P5BIT || fmt == VQKV_FMT_3BIT || fmt == VQKV_FMT_1P25BIT ||
           fmt == VQKV_FMT_4BIT;
}

// Checks shared by every call that takes a shape.  `need_cache` adds the
// capacity and format checks.
vqkv_status check_shape(const vqkv_shape* s, bool need_cache) {
    if (!s) return fail(VQKV_ERR_INVALID_ARG, "shape is NULL");
    if (s->head_dim != 128) return fail(VQKV_ERR_UNSUPPORTED, "head_dim %d unsupported (must be 128)", s->head_dim);
    if (s->batch < 1) return fail(VQKV_ERR_INVALID_ARG, "batch %d < 1", s->batch);
    if (s->num_q_heads < 1 || s->num_kv_heads < 1)
        return fail(VQKV_ERR_INVALID_ARG, "head counts must be >= 1 (Hq %d, Hkv %d)", s->num_q_heads, s->num_kv_heads);
    if (s->num_q_heads % s->num_kv_heads != 0)
        return fail(VQKV_ERR_INVALID_ARG, "Hq %d is not a multiple of Hkv %d", s->num_q_heads, s->num_kv_heads);
    const int G = s->num_q_heads / s->num_kv_heads;
    if (G > 8) return fail(VQKV_ERR_UNSUPPORTED, "group size Hq/Hkv = %d exceeds 8", G);
    if ((int64_t)s->batch * s->num_q_heads > (1 << 24))
        return fail(VQKV_ERR_UNSUPPORTED, "batch * Hq too large");
    if (need_cache) {
        if (!known_fmt(base_fmt(s->fmt)) ||
            (s->fmt & ~(0xff | VQKV_FMT_VALUE_TRANSFORM)) != 0)
            return fail(VQKV_ERR_INVALID_ARG, "unknown format %d", s->fmt);
        if (s->max_tokens < 64 || s->max_tokens % 64 != 0)
            return fail(VQKV_ERR_INVALID_ARG, "max_tokens %d must be a positive multiple of 64", s->max_tokens);
    }
    return VQKV_OK;
}

#define VQKV_CHECK(expr)                         \
    do {                                         \
        vqkv_status _st = (expr);                \
        if (_st != VQKV_OK) return _st;          \
    } while (0)

vqkv_status check_ptr(const void* p, const char* name) {
    if (!p) return fail(VQKV_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(VQKV_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return VQKV_OK;
}

vqkv_status check_dtype(int32_t dt) {
    if (dt != VQKV_DTYPE_BF16 && dt != VQKV_DTYPE_FP32) return fail(VQKV_ERR_INVALID_ARG, "unknown dtype %d", dt);
    return VQKV_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Token range per split: 64-aligned, covering [0, seq_len) with `splits` ranges.
int split_chunk(int seq_len, int splits) {
    const int64_t tiles = ceil_div(seq_len, 64);
    return (int)(ceil_div(tiles, splits) * 64);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units of the current device (the decode kernels keep one
// work-group per CU); 256, an MI355X's count, when no device answers.
int compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
    return n;
}


}  // namespace

extern "C" {

size_t vqkv_code_bytes_per_token(int32_t fmt) {
    if ((fmt & ~(0xff | VQKV_FMT_VALUE_TRANSFORM)) != 0) return 0;
    if (base_fmt(fmt) == VQKV_FMT_2BIT) return 32;
    if (base_fmt(fmt) == VQKV_FMT_1P5BIT) return 24;
    if (base_fmt(fmt) == VQKV_FMT_3BIT) return 48;
    if (base_fmt(fmt) == VQKV_FMT_1P25BIT) return 20;
    if (base_fmt(fmt) == VQKV_FMT_4BIT) return 64;
    return 0;
}

size_t vqkv_cache_bytes(const vqkv_shape* s) {
    if (check_shape(s, true) != VQKV_OK) return 0;
    return (size_t)s->batch * s->num_kv_heads * s->max_tokens * vqkv_code_bytes_per_token(s->fmt);
}

size_t vqkv_workspace_bytes(const vqkv_shape* s, int32_t num_splits) {
    if (check_shape(s, false) != VQKV_OK || num_splits < 1) return 0;
    const size_t rows = (size_t)s->batch * s->num_q_heads * num_splits;
    return align256(rows * 128 * sizeof(float)) + align256(rows * 2 * sizeof(float));
}

size_t vqkv_step_workspace_bytes(const vqkv_shape* s, int32_t num_splits) {
    const size_t base = vqkv_workspace_bytes(s, num_splits);
    if (base == 0) return 0;
    return base + align256((size_t)s->batch * s->num_q_heads * 128 * sizeof(float)) +
           align256((size_t)s->batch * s->num_kv_heads * sizeof(int32_t)) +
           align256((size_t)s->batch * sizeof(int32_t));
}

int32_t vqkv_suggest_splits(const vqkv_shape* s, int32_t seq_len) {
    if (check_shape(s, false) != VQKV_OK || seq_len < 1) return 1;
    const int64_t streams = (int64_t)s->batch * s->num_kv_heads;
    const int64_t want = ceil_div(compute_units(), streams);  // one work-group per CU
    const int64_t cap = ceil_div(seq_len, 1024);              // keep >= 1024 tokens per split
    int64_t S = want < cap ? want : cap;
    if (S < 1) S = 1;
    return (int32_t)S;
}

const char* vqkv_status_string(int32_t st) {
    switch (st) {
        case VQKV_OK: return "ok";
        case VQKV_ERR_INVALID_ARG: return "invalid argument";
        case VQKV_ERR_UNSUPPORTED: return "unsupported";
        case VQKV_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* vqkv_last_error(void) { return g_last_error; }

vqkv_status vqkv_transform_query(const vqkv_shape* s, const void* q, int32_t q_dtype, const float* smooth,
                                 float* q_prime, void* stream) {
    VQKV_CHECK(check_shape(s, false));
    VQKV_CHECK(check_dtype(q_dtype));
    VQKV_CHECK(check_ptr(q, "q"));
    VQKV_CHECK(check_ptr(smooth, "smooth"));
    VQKV_CHECK(check_ptr(q_prime, "q_prime"));
    vqkv::TransformQueryArgs a{q, q_dtype, smooth, q_prime, s->batch, s->num_q_heads, s->num_kv_heads};
    return hip_status(vqkv::launch_transform_query(a, (hipStream_t)stream), "transform_query launch");
}

vqkv_status vqkv_quantize_append(const vqkv_shape* s, const void* k_new, const void* v_new, int32_t dtype,
                                 int32_t n_new, int32_t start_pos, const float* smooth, const uint16_t* k_book,
                                 const uint16_t* v_book, uint8_t* k_codes, uint8_t* v_codes, void* stream) {
    VQKV_CHECK(check_shape(s, true));
    VQKV_CHECK(check_dtype(dtype));
    if (n_new < 1) return fail(VQKV_ERR_INVALID_ARG, "n_new %d < 1", n_new);
    if (start_pos < 0) return fail(VQKV_ERR_INVALID_ARG, "start_pos %d < 0", start_pos);
    if ((int64_t)start_pos + n_new > s->max_tokens)
        return fail(VQKV_ERR_INVALID_ARG, "start_pos + n_new = %lld exceeds max_tokens %d",
                    (long long)start_pos + n_new, s->max_tokens);
    VQKV_CHECK(check_ptr(k_new, "k_new"));
    VQKV_CHECK(check_ptr(v_new, "v_new"));
    VQKV_CHECK(check_ptr(smooth, "smooth"));
    VQKV_CHECK(check_ptr(k_book, "k_book"));
    VQKV_CHECK(check_ptr(v_book, "v_book"));
    VQKV_CHECK(check_ptr(k_codes, "k_codes"));
    VQKV_CHECK(check_ptr(v_codes, "v_codes"));
    vqkv::AppendArgs a{k_new, v_new, dtype, n_new, start_pos, smooth, k_book, v_book, k_codes, v_codes,
                       s->batch, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt)};
    a.v_smooth = value_scales(s, smooth);
    return hip_status(vqkv::launch_quantize_append(a, (hipStream_t)stream), "quantize_append launch");
}

vqkv_status vqkv_quantize_append_varlen(const vqkv_shape* s, const void* k_new, const void* v_new, int32_t dtype,
                                        const int32_t* positions, const float* smooth, const uint16_t* k_book,
                                        const uint16_t* v_book, uint8_t* k_codes, uint8_t* v_codes, void* stream) {
    VQKV_CHECK(check_shape(s, true));
    VQKV_CHECK(check_dtype(dtype));
    if (!positions) return fail(VQKV_ERR_INVALID_ARG, "positions is NULL");
    if ((uintptr_t)positions & 3) return fail(VQKV_ERR_INVALID_ARG, "positions is not 4-byte aligned");
    VQKV_CHECK(check_ptr(k_new, "k_new"));
    VQKV_CHECK(check_ptr(v_new, "v_new"));
    VQKV_CHECK(check_ptr(smooth, "smooth"));
    VQKV_CHECK(check_ptr(k_book, "k_book"));
    VQKV_CHECK(check_ptr(v_book, "v_book"));
    VQKV_CHECK(check_ptr(k_codes, "k_codes"));
    VQKV_CHECK(check_ptr(v_codes, "v_codes"));
    vqkv::AppendArgs a{k_new, v_new, dtype, 1, 0, smooth, k_book, v_book, k_codes, v_codes,
                       s->batch, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt), positions};
    a.v_smooth = value_scales(s, smooth);
    return hip_status(vqkv::launch_quantize_append(a, (hipStream_t)stream), "quantize_append_varlen launch");
}

vqkv_status vqkv_quantize_append_paged(const vqkv_shape* s, const void* k_new, const void* v_new, int32_t dtype,
                                       const int32_t* positions, const float* smooth, const uint16_t* k_book,
                                       const uint16_t* v_book, uint8_t* k_pool, uint8_t* v_pool, int32_t num_blocks,
                                       const int32_t* block_table, void* stream) {
    VQKV_CHECK(check_shape(s, true));
    VQKV_CHECK(check_dtype(dtype));
    if (num_blocks < 1) return fail(VQKV_ERR_INVALID_ARG, "num_blocks %d < 1", num_blocks);
    if (!block_table) return fail(VQKV_ERR_INVALID_ARG, "block_table is NULL");
    if ((uintptr_t)block_table & 3) return fail(VQKV_ERR_INVALID_ARG, "block_table is not 4-byte aligned");
    if (!positions) return fail(VQKV_ERR_INVALID_ARG, "positions is NULL");
    if ((uintptr_t)positions & 3) return fail(VQKV_ERR_INVALID_ARG, "positions is not 4-byte aligned");
    VQKV_CHECK(check_ptr(k_new, "k_new"));
    VQKV_CHECK(check_ptr(v_new, "v_new"));
    VQKV_CHECK(check_ptr(smooth, "smooth"));
    VQKV_CHECK(check_ptr(k_book, "k_book"));
    VQKV_CHECK(check_ptr(v_book, "v_book"));
    VQKV_CHECK(check_ptr(k_pool, "k_pool"));
    VQKV_CHECK(check_ptr(v_pool, "v_pool"));
    vqkv::AppendArgs a{k_new, v_new, dtype, 1, 0, smooth, k_book, v_book, k_pool, v_pool,
                       s->batch, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt), positions, block_table, num_blocks};
    a.v_smooth = value_scales(s, smooth);
    return hip_status(vqkv::launch_quantize_append(a, (hipStream_t)stream), "quantize_append_paged launch");
}

}  // extern "C"

namespace {

// vqkv_decode_attention on a chosen kernel: 0 the default (matrix cores),
// 1 score table, 2 gather, 3 matrix cores named explicitly.
vqkv_status decode_attention_impl(const vqkv_shape* s, const float* q_prime, const uint16_t* k_book,
                                  const uint16_t* v_book, const uint8_t* k_codes, const uint8_t* v_codes,
                                  int32_t seq_len, float sm_scale, int32_t num_splits, void* workspace,
                                  int path, void* stream) {
    VQKV_CHECK(check_shape(s, true));
    if (seq_len < 1 || seq_len > s->max_tokens)
        return fail(VQKV_ERR_INVALID_ARG, "seq_len %d outside [1, max_tokens = %d]", seq_len, s->max_tokens);
    if (!std::isfinite(sm_scale)) return fail(VQKV_ERR_INVALID_ARG, "sm_scale is not finite");
    if (num_splits < 1 || num_splits > ceil_div(seq_len, 64))
        return fail(VQKV_ERR_INVALID_ARG, "num_splits %d outside [1, ceil(seq_len / 64) = %lld]", num_splits,
                    (long long)ceil_div(seq_len, 64));
    VQKV_CHECK(check_ptr(q_prime, "q_prime"));
    VQKV_CHECK(check_ptr(k_book, "k_book"));
    VQKV_CHECK(check_ptr(v_book, "v_book"));
    VQKV_CHECK(check_ptr(k_codes, "k_codes"));
    VQKV_CHECK(check_ptr(v_codes, "v_codes"));
    VQKV_CHECK(check_ptr(workspace, "workspace"));
    const size_t rows = (size_t)s->batch * s->num_q_heads * num_splits;
    float* part_o = (float*)workspace;
    float* part_ml = (float*)((char*)workspace + align256(rows * 128 * sizeof(float)));
    const int G = s->num_q_heads / s->num_kv_heads;
    if (path < 0 || path > 3) return fail(VQKV_ERR_INVALID_ARG, "unknown decode path %d", path);
    if (path == 1 && !(base_fmt(s->fmt) == VQKV_FMT_2BIT && G <= 4))
        return fail(VQKV_ERR_UNSUPPORTED, "score-table path needs the 2-bit format and Hq/Hkv <= 4");
    if (path == 2 && base_fmt(s->fmt) != VQKV_FMT_2BIT && base_fmt(s->fmt) != VQKV_FMT_1P5BIT)
        return fail(VQKV_ERR_UNSUPPORTED, "the gather path takes the 2-bit and 1.5-bit formats");
    vqkv::DecodeArgs a{q_prime, k_book, v_book, k_codes, v_codes, part_o, part_ml,
                       s->batch, s->num_q_heads, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt),
                       seq_len, num_splits, split_chunk(seq_len, num_splits),
                       (float)((double)sm_scale * 1.4426950408889634), path};
    return hip_status(vqkv::launch_decode(a, (hipStream_t)stream), "decode_attention launch");
}

}  // namespace

extern "C" {

vqkv_status vqkv_decode_attention(const vqkv_shape* s, const float* q_prime, const uint16_t* k_book,
                                  const uint16_t* v_book, const uint8_t* k_codes, const uint8_t* v_codes,
                                  int32_t seq_len, float sm_scale, int32_t num_splits, void* workspace,
                                  void* stream) {
    return decode_attention_impl(s, q_prime, k_book, v_book, k_codes, v_codes, seq_len, sm_scale, num_splits,
                                 workspace, 0, stream);
}

vqkv_status vqkv_measure_decode_attention(const vqkv_shape* s, const float* q_prime, const uint16_t* k_book,
                                          const uint16_t* v_book, const uint8_t* k_codes, const uint8_t* v_codes,
                                          int32_t seq_len, float sm_scale, int32_t num_splits, void* workspace,
                                          int32_t path, void* stream) {
    return decode_attention_impl(s, q_prime, k_book, v_book, k_codes, v_codes, seq_len, sm_scale, num_splits,
                                 workspace, path, stream);
}

vqkv_status vqkv_decode_attention_varlen(const vqkv_shape* s, const float* q_prime, const uint16_t* k_book,
                                         const uint16_t* v_book, const uint8_t* k_codes, const uint8_t* v_codes,
                                         const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                         int32_t num_splits, void* workspace, void* stream) {
    VQKV_CHECK(check_shape(s, true));
    if (max_seq_len < 1 || max_seq_len > s->max_tokens)
        return fail(VQKV_ERR_INVALID_ARG, "max_seq_len %d outside [1, max_tokens = %d]", max_seq_len, s->max_tokens);
    if (!seq_lens) return fail(VQKV_ERR_INVALID_ARG, "seq_lens is NULL");
    if ((uintptr_t)seq_lens & 3) return fail(VQKV_ERR_INVALID_ARG, "seq_lens is not 4-byte aligned");
    if (!std::isfinite(sm_scale)) return fail(VQKV_ERR_INVALID_ARG, "sm_scale is not finite");
    if (num_splits < 1 || num_splits > ceil_div(max_seq_len, 64))
        return fail(VQKV_ERR_INVALID_ARG, "num_splits %d outside [1, ceil(max_seq_len / 64) = %lld]", num_splits,
                    (long long)ceil_div(max_seq_len, 64));
    VQKV_CHECK(check_ptr(q_prime, "q_prime"));
    VQKV_CHECK(check_ptr(k_book, "k_book"));
    VQKV_CHECK(check_ptr(v_book, "v_book"));
    VQKV_CHECK(check_ptr(k_codes, "k_codes"));
    VQKV_CHECK(check_ptr(v_codes, "v_codes"));
    VQKV_CHECK(check_ptr(workspace, "workspace"));
    const size_t rows = (size_t)s->batch * s->num_q_heads * num_splits;
    float* part_o = (float*)workspace;
    float* part_ml = (float*)((char*)workspace + align256(rows * 128 * sizeof(float)));
    vqkv::DecodeArgs a{q_prime, k_book, v_book, k_codes, v_codes, part_o, part_ml,
                       s->batch, s->num_q_heads, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt),
                       max_seq_len, num_splits, split_chunk(max_seq_len, num_splits),
                       (float)((double)sm_scale * 1.4426950408889634), 0, seq_lens};
    return hip_status(vqkv::launch_decode(a, (hipStream_t)stream), "decode_attention_varlen launch");
}

vqkv_status vqkv_decode_attention_paged(const vqkv_shape* s, const float* q_prime, const uint16_t* k_book,
                                        const uint16_t* v_book, const uint8_t* k_pool, const uint8_t* v_pool,
                                        int32_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                                        int32_t max_seq_len, float sm_scale, int32_t num_splits, void* workspace,
                                        void* stream) {
    VQKV_CHECK(check_shape(s, true));
    if (num_blocks < 1) return fail(VQKV_ERR_INVALID_ARG, "num_blocks %d < 1", num_blocks);
    if (!block_table) return fail(VQKV_ERR_INVALID_ARG, "block_table is NULL");
    if ((uintptr_t)block_table & 3) return fail(VQKV_ERR_INVALID_ARG, "block_table is not 4-byte aligned");
    if (max_seq_len < 1 || max_seq_len > s->max_tokens)
        return fail(VQKV_ERR_INVALID_ARG, "max_seq_len %d outside [1, max_tokens = %d]", max_seq_len, s->max_tokens);
    if (!seq_lens) return fail(VQKV_ERR_INVALID_ARG, "seq_lens is NULL");
    if ((uintptr_t)seq_lens & 3) return fail(VQKV_ERR_INVALID_ARG, "seq_lens is not 4-byte aligned");
    if (!std::isfinite(sm_scale)) return fail(VQKV_ERR_INVALID_ARG, "sm_scale is not finite");
    if (num_splits < 1 || num_splits > ceil_div(max_seq_len, 64))
        return fail(VQKV_ERR_INVALID_ARG, "num_splits %d outside [1, ceil(max_seq_len / 64) = %lld]", num_splits,
                    (long long)ceil_div(max_seq_len, 64));
    VQKV_CHECK(check_ptr(q_prime, "q_prime"));
    VQKV_CHECK(check_ptr(k_book, "k_book"));
    VQKV_CHECK(check_ptr(v_book, "v_book"));
    VQKV_CHECK(check_ptr(k_pool, "k_pool"));
    VQKV_CHECK(check_ptr(v_pool, "v_pool"));
    VQKV_CHECK(check_ptr(workspace, "workspace"));
    const size_t rows = (size_t)s->batch * s->num_q_heads * num_splits;
    float* part_o = (float*)workspace;
    float* part_ml = (float*)((char*)workspace + align256(rows * 128 * sizeof(float)));
    vqkv::DecodeArgs a{q_prime, k_book, v_book, k_pool, v_pool, part_o, part_ml,
                       s->batch, s->num_q_heads, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt),
                       max_seq_len, num_splits, split_chunk(max_seq_len, num_splits),
                       (float)((double)sm_scale * 1.4426950408889634), 0, seq_lens, block_table, num_blocks};
    return hip_status(vqkv::launch_decode(a, (hipStream_t)stream), "decode_attention_paged launch");
}

}  // extern "C"

namespace {

// The fused step for every cache form: uniform position (positions null), or
// one position per sequence, with (block_table) or without a block pool.
vqkv_status decode_step_impl(const vqkv_shape* s, const void* q, const void* k_new, const void* v_new,
                             int32_t dtype, int32_t position, const int32_t* positions, int32_t max_seq_len,
                             const float* smooth, const uint16_t* k_book, const uint16_t* v_book,
                             uint8_t* k_codes, uint8_t* v_codes, int32_t num_blocks, const int32_t* block_table,
                             float sm_scale, int32_t num_splits, void* workspace, float* out, void* stream,
                             const char* name) {
    VQKV_CHECK(check_shape(s, true));
    VQKV_CHECK(check_dtype(dtype));
    int seq_len;
    if (positions == nullptr) {
        if (position < 0 || position >= s->max_tokens)
            return fail(VQKV_ERR_INVALID_ARG, "position %d outside [0, max_tokens = %d)", position, s->max_tokens);
        seq_len = position + 1;
    } else {
        if ((uintptr_t)positions & 3) return fail(VQKV_ERR_INVALID_ARG, "positions is not 4-byte aligned");
        if (max_seq_len < 1 || max_seq_len > s->max_tokens)
            return fail(VQKV_ERR_INVALID_ARG, "max_seq_len %d outside [1, max_tokens = %d]", max_seq_len,
                        s->max_tokens);
        seq_len = max_seq_len;
    }
    if (block_table != nullptr) {
        if (num_blocks < 1) return fail(VQKV_ERR_INVALID_ARG, "num_blocks %d < 1", num_blocks);
        if ((uintptr_t)block_table & 3) return fail(VQKV_ERR_INVALID_ARG, "block_table is not 4-byte aligned");
    }
    if (!std::isfinite(sm_scale)) return fail(VQKV_ERR_INVALID_ARG, "sm_scale is not finite");
    if (num_splits < 1 || num_splits > ceil_div(seq_len, 64))
        return fail(VQKV_ERR_INVALID_ARG, "num_splits %d outside [1, ceil(%d / 64) = %lld]", num_splits, seq_len,
                    (long long)ceil_div(seq_len, 64));
    VQKV_CHECK(check_ptr(q, "q"));
    VQKV_CHECK(check_ptr(k_new, "k_new"));
    VQKV_CHECK(check_ptr(v_new, "v_new"));
    VQKV_CHECK(check_ptr(smooth, "smooth"));
    VQKV_CHECK(check_ptr(k_book, "k_book"));
    VQKV_CHECK(check_ptr(v_book, "v_book"));
    VQKV_CHECK(check_ptr(k_codes, "k_codes"));
    VQKV_CHECK(check_ptr(v_codes, "v_codes"));
    VQKV_CHECK(check_ptr(workspace, "workspace"));
    VQKV_CHECK(check_ptr(out, "out"));
    // Workspace: partial o | partial (m, ll) pairs | q' | arrival counters | sequence lengths.
    const size_t rows = (size_t)s->batch * s->num_q_heads * num_splits;
    char* ws = (char*)workspace;
    float* part_o = (float*)ws;
    ws += align256(rows * 128 * sizeof(float));
    float* part_ml = (float*)ws;
    ws += align256(rows * 2 * sizeof(float));
    float* q_prime = (float*)ws;
    ws += align256((size_t)s->batch * s->num_q_heads * 128 * sizeof(float));
    int32_t* arrivals = (int32_t*)ws;
    ws += align256((size_t)s->batch * s->num_kv_heads * sizeof(int32_t));
    int32_t* seq_lens = positions ? (int32_t*)ws : nullptr;
    vqkv::AppendArgs ap{k_new, v_new, dtype, 1, positions ? 0 : position, smooth, k_book, v_book, k_codes,
                        v_codes, s->batch, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt), positions, block_table,
                        num_blocks, q, q_prime, arrivals, s->num_q_heads, seq_lens};
    char what[64];
    ap.v_smooth = value_scales(s, smooth);
    vqkv::DecodeArgs d{q_prime, k_book, v_book, k_codes, v_codes, part_o, part_ml,
                       s->batch, s->num_q_heads, s->num_kv_heads, s->max_tokens, base_fmt(s->fmt),
                       seq_len, num_splits, split_chunk(seq_len, num_splits),
                       (float)((double)sm_scale * 1.4426950408889634), 3, seq_lens, block_table, num_blocks,
                       out, arrivals, value_scales(s, smooth)};
    if (base_fmt(s->fmt) == 0 && num_splits == 1) {
        // One launch: each work-group appends its own head's token before its
        // pass (nothing to combine with one split, so no counters either).
        d.q_prime = nullptr;
        d.seq_lens = nullptr;
        d.app = ap;
        snprintf(what, sizeof(what), "%s fused decode launch", name);
        return hip_status(vqkv::launch_decode(d, (hipStream_t)stream), what);
    }
    if (base_fmt(s->fmt) == 0 && ap.v_smooth == nullptr) {
        // Two launches: the attention kernel appends the token in the work-group
        // whose split holds it (every work-group transforms its query heads) and
        // writes the splits' partials, then the combine kernel merges them (no
        // arrival counters).
        d.q_prime = nullptr;
        d.seq_lens = nullptr;
        d.app = ap;
        d.out = nullptr;
        snprintf(what, sizeof(what), "%s fused decode launch", name);
        VQKV_CHECK(hip_status(vqkv::launch_decode(d, (hipStream_t)stream), what));
        vqkv::CombineArgs c{part_o, part_ml, out, s->batch, s->num_q_heads, num_splits};
        snprintf(what, sizeof(what), "%s combine launch", name);
        return hip_status(vqkv::launch_combine(c, (hipStream_t)stream), what);
    }
    snprintf(what, sizeof(what), "%s append launch", name);
    VQKV_CHECK(hip_status(vqkv::launch_quantize_append(ap, (hipStream_t)stream), what));
    if (num_splits > 1 && ap.v_smooth == nullptr) {
        // Three launches: the attention writes the splits' partials and the
        // combine kernel merges them (2-2.5 us shorter per step than the last
        // split of each head combining after a release/acquire pair, for the
        // 1.5-, 1.25-, 3- and 4-bit batch-8 steps).
        d.out = nullptr;
        snprintf(what, sizeof(what), "%s decode launch", name);
        VQKV_CHECK(hip_status(vqkv::launch_decode(d, (hipStream_t)stream), what));
        vqkv::CombineArgs c{part_o, part_ml, out, s->batch, s->num_q_heads, num_splits};
        snprintf(what, sizeof(what), "%s combine launch", name);
        return hip_status(vqkv::launch_combine(c, (hipStream_t)stream), what);
    }
    snprintf(what, sizeof(what), "%s decode launch", name);
    return hip_status(vqkv::launch_decode(d, (hipStream_t)stream), what);
}

}  // namespace

extern "C" {

vqkv_status vqkv_decode_step(const vqkv_shape* s, const void* q, const void* k_new, const void* v_new,
                             int32_t dtype, int32_t position, const float* smooth, const uint16_t* k_book,
                             const uint16_t* v_book, uint8_t* k_codes, uint8_t* v_codes, float sm_scale,
                             int32_t num_splits, void* workspace, float* out, void* stream) {
    return decode_step_impl(s, q, k_new, v_new, dtype, position, nullptr, 0, smooth, k_book, v_book, k_codes,
                            v_codes, 0, nullptr, sm_scale, num_splits, workspace, out, stream, "decode_step");
}

vqkv_status vqkv_decode_step_static(const vqkv_shape* s, const void* q, const void* k_new, const void* v_new,
                                    int32_t dtype, int32_t position, const float* smooth, const uint16_t* k_book,
                                    const uint16_t* v_book, uint8_t* k_codes, uint8_t* v_codes, float sm_scale,
                                    int32_t num_splits, float* out, void* stream) {
    static_assert(VQKV_STATIC_SCRATCH_BYTES == vqkv::kStaticScratchBytes, "one size in the header and the library");
    VQKV_CHECK(check_shape(s, true));
    if (num_splits < 1) return fail(VQKV_ERR_INVALID_ARG, "num_splits %d < 1", num_splits);
    const size_t need = vqkv_step_workspace_bytes(s, num_splits);
    if (need > vqkv::kStaticScratchBytes)
        return fail(VQKV_ERR_UNSUPPORTED, "the step needs %zu bytes of workspace, more than the %zu bytes of the "
                    "static scratch (use vqkv_decode_step with a workspace)", need, vqkv::kStaticScratchBytes);
    void* ws = nullptr;
    VQKV_CHECK(hip_status(vqkv::static_scratch(&ws, nullptr), "static scratch address"));
    return decode_step_impl(s, q, k_new, v_new, dtype, position, nullptr, 0, smooth, k_book, v_book, k_codes,
                            v_codes, 0, nullptr, sm_scale, num_splits, ws, out, stream, "decode_step_static");
}

vqkv_status vqkv_decode_step_varlen(const vqkv_shape* s, const void* q, const void* k_new, const void* v_new,
                                    int32_t dtype, const int32_t* positions, int32_t max_seq_len,
                                    const float* smooth, const uint16_t* k_book, const uint16_t* v_book,
                                    uint8_t* k_codes, uint8_t* v_codes, float sm_scale, int32_t num_splits,
                                    void* workspace, float* out, void* stream) {
    if (!positions) return fail(VQKV_ERR_INVALID_ARG, "positions is NULL");
    return decode_step_impl(s, q, k_new, v_new, dtype, 0, positions, max_seq_len, smooth, k_book, v_book,
                            k_codes, v_codes, 0, nullptr, sm_scale, num_splits, workspace, out, stream,
                            "decode_step_varlen");
}

vqkv_status vqkv_decode_step_paged(const vqkv_shape* s, const void* q, const void* k_new, const void* v_new,
                                   int32_t dtype, const int32_t* positions, int32_t max_seq_len,
                                   const float* smooth, const uint16_t* k_book, const uint16_t* v_book,
                                   uint8_t* k_pool, uint8_t* v_pool, int32_t num_blocks,
                                   const int32_t* block_table, float sm_scale, int32_t num_splits,
                                   void* workspace, float* out, void* stream) {
    if (!positions) return fail(VQKV_ERR_INVALID_ARG, "positions is NULL");
    if (!block_table) return fail(VQKV_ERR_INVALID_ARG, "block_table is NULL");
    return decode_step_impl(s, q, k_new, v_new, dtype, 0, positions, max_seq_len, smooth, k_book, v_book,
                            k_pool, v_pool, num_blocks, block_table, sm_scale, num_splits, workspace, out,
                            stream, "decode_step_paged");
}

vqkv_status vqkv_combine(const vqkv_shape* s, int32_t num_splits, const void* workspace, float* out, void* stream) {
    VQKV_CHECK(check_shape(s, false));
    if (num_splits < 1) return fail(VQKV_ERR_INVALID_ARG, "num_splits %d < 1", num_splits);
    VQKV_CHECK(check_ptr(workspace, "workspace"));
    VQKV_CHECK(check_ptr(out, "out"));
    const size_t rows = (size_t)s->batch * s->num_q_heads * num_splits;
    const float* part_o = (const float*)workspace;
    const float* part_ml = (const float*)((const char*)workspace + align256(rows * 128 * sizeof(float)));
    vqkv::CombineArgs a{part_o, part_ml, out, s->batch, s->num_q_heads, num_splits};
    return hip_status(vqkv::launch_combine(a, (hipStream_t)stream), "combine launch");
}

vqkv_status vqkv_value_output_transform(const vqkv_shape* s, const float* smooth, float* out, void* stream) {
    VQKV_CHECK(check_shape(s, true));
    if (!(s->fmt & VQKV_FMT_VALUE_TRANSFORM))
        return fail(VQKV_ERR_INVALID_ARG, "the shape's format has no value transform to undo");
    VQKV_CHECK(check_ptr(smooth, "smooth"));
    VQKV_CHECK(check_ptr(out, "out"));
    vqkv::ValueOutputArgs a{out, value_scales(s, smooth), s->batch, s->num_q_heads, s->num_kv_heads};
    return hip_status(vqkv::launch_value_output_transform(a, (hipStream_t)stream), "value_output_transform launch");
}

vqkv_status vqkv_smooth_scales(int32_t num_kv_heads, int32_t n_cal, const void* k_cal, int32_t dtype,
                               float* smooth, void* stream) {
    if (num_kv_heads < 1) return fail(VQKV_ERR_INVALID_ARG, "num_kv_heads %d < 1", num_kv_heads);
    if (n_cal < 1) return fail(VQKV_ERR_INVALID_ARG, "n_cal %d < 1", n_cal);
    VQKV_CHECK(check_dtype(dtype));
    VQKV_CHECK(check_ptr(k_cal, "k_cal"));
    VQKV_CHECK(check_ptr(smooth, "smooth"));
    return hip_status(vqkv::launch_smooth_scales(num_kv_heads, n_cal, k_cal, dtype, smooth, (hipStream_t)stream),
                      "smooth_scales launch");
}

size_t vqkv_train_workspace_bytes(int32_t fmt, int32_t n_cal) {
    if (!known_fmt(fmt) || n_cal < 1) return 0;
    const size_t n_pts = (size_t)n_cal * (128 / dsub_of(fmt));
    return align256((size_t)n_cal * 128 * sizeof(double)) + align256(n_pts * sizeof(int32_t)) +
           align256((size_t)entries_of(fmt) * dsub_of(fmt) * sizeof(double));
}

vqkv_status vqkv_train_codebook(int32_t fmt, int32_t n_cal, const void* rows, int32_t dtype, int32_t is_key,
                                const float* smooth, const int64_t* init_idx, int32_t iters, uint16_t* book,
                                double* centroids, void* workspace, void* stream) {
    if (!known_fmt(fmt)) return fail(VQKV_ERR_INVALID_ARG, "unknown format %d", fmt);
    const int E = entries_of(fmt);
    const int64_t n_pts = (int64_t)n_cal * (128 / dsub_of(fmt));
    if (n_cal < 1 || n_pts < E)
        return fail(VQKV_ERR_INVALID_ARG, "n_cal %d gives %lld points, fewer than %d entries", n_cal,
                    (long long)n_pts, E);
    if (n_cal > (1 << 22)) return fail(VQKV_ERR_UNSUPPORTED, "n_cal %d too large", n_cal);
    if (iters < 0) return fail(VQKV_ERR_INVALID_ARG, "iters %d < 0", iters);
    VQKV_CHECK(check_dtype(dtype));
    VQKV_CHECK(check_ptr(rows, "rows"));
    if (is_key) VQKV_CHECK(check_ptr(smooth, "smooth"));
    VQKV_CHECK(check_ptr(init_idx, "init_idx"));
    VQKV_CHECK(check_ptr(book, "book"));
    if (centroids) VQKV_CHECK(check_ptr(centroids, "centroids"));
    VQKV_CHECK(check_ptr(workspace, "workspace"));
    char* ws = (char*)workspace;
    double* points = (double*)ws;
    ws += align256((size_t)n_cal * 128 * sizeof(double));
    int32_t* assign = (int32_t*)ws;
    ws += align256((size_t)n_pts * sizeof(int32_t));
    double* cent = centroids ? centroids : (double*)ws;
    vqkv::TrainArgs a{fmt, n_cal, dtype, is_key, iters, rows, smooth, init_idx, book, cent, points, assign};
    return hip_status(vqkv::launch_train_codebook(a, (hipStream_t)stream), "train_codebook launch");
}

}  // extern "C"
