// Drives the C ABI's host code (built with stub launchers) under the
// sanitizers: every rejected argument returns its status without a launch,
// and well-formed calls pass the checks and reach exactly the expected
// launches.  Pointers are aligned dummies; nothing dereferences them.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "../../include/vqkv.h"

extern int g_launches;

#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main() {
    auto P = [](uintptr_t a) { return reinterpret_cast<void*>(a); };
    void* F = P(0x10000);
    float* Ff = static_cast<float*>(F);
    const uint16_t* Fb = static_cast<const uint16_t*>(F);
    uint8_t* Fc = static_cast<uint8_t*>(F);
    const int32_t* Fi = static_cast<const int32_t*>(F);
    vqkv_shape good{32, 32, 8, 128, 196608, VQKV_FMT_2BIT};
    for (int fmt : {(int)VQKV_FMT_2BIT, (int)VQKV_FMT_1P5BIT, (int)VQKV_FMT_3BIT, (int)VQKV_FMT_1P25BIT,
                    (int)VQKV_FMT_4BIT, (int)VQKV_FMT_3BIT | (int)VQKV_FMT_VALUE_TRANSFORM}) {
        vqkv_shape s = good;
        s.fmt = fmt;
        CHECK(vqkv_cache_bytes(&s) > 0);
        CHECK(vqkv_workspace_bytes(&s, 3) > 0 && vqkv_step_workspace_bytes(&s, 3) > vqkv_workspace_bytes(&s, 3));
        int before = g_launches;
        CHECK(vqkv_transform_query(&s, F, 0, Ff, Ff, nullptr) == VQKV_OK);
        CHECK(vqkv_quantize_append(&s, F, F, 0, 5, 100, Ff, Fb, Fb, Fc, Fc, nullptr) == VQKV_OK);
        CHECK(vqkv_quantize_append_varlen(&s, F, F, 0, Fi, Ff, Fb, Fb, Fc, Fc, nullptr) == VQKV_OK);
        CHECK(vqkv_quantize_append_paged(&s, F, F, 0, Fi, Ff, Fb, Fb, Fc, Fc, 7, Fi, nullptr) == VQKV_OK);
        CHECK(vqkv_decode_attention(&s, Ff, Fb, Fb, Fc, Fc, 4099, 0.088f, 9, F, nullptr) == VQKV_OK);
        CHECK(vqkv_decode_attention_varlen(&s, Ff, Fb, Fb, Fc, Fc, Fi, 4099, 0.088f, 9, F, nullptr) == VQKV_OK);
        CHECK(vqkv_decode_attention_paged(&s, Ff, Fb, Fb, Fc, Fc, 7, Fi, Fi, 4099, 0.088f, 9, F, nullptr) == VQKV_OK);
        CHECK(vqkv_combine(&s, 9, F, Ff, nullptr) == VQKV_OK);
        CHECK(vqkv_decode_step(&s, F, F, F, 0, 4098, Ff, Fb, Fb, Fc, Fc, 0.088f, 9, F, Ff, nullptr) == VQKV_OK);
        CHECK(vqkv_decode_step_varlen(&s, F, F, F, 0, Fi, 4099, Ff, Fb, Fb, Fc, Fc, 0.088f, 9, F, Ff, nullptr) == VQKV_OK);
        CHECK(vqkv_decode_step_paged(&s, F, F, F, 0, Fi, 4099, Ff, Fb, Fb, Fc, Fc, 7, Fi, 0.088f, 9, F, Ff, nullptr) == VQKV_OK);
        CHECK(vqkv_decode_step_static(&s, F, F, F, 0, 4098, Ff, Fb, Fb, Fc, Fc, 0.088f, 1, Ff, nullptr) == VQKV_OK);
        const int vt = (fmt & VQKV_FMT_VALUE_TRANSFORM) != 0;
        CHECK(vqkv_value_output_transform(&s, Ff, Ff, nullptr) == (vt ? VQKV_OK : VQKV_ERR_INVALID_ARG));
        // Steps at 9 splits: 2-bit, fused append + combine (2); the value transform, append + attention
        // with the fused combine (2); the other formats, append + attention + combine (3).
        const int step_launches = (fmt == VQKV_FMT_2BIT || vt) ? 2 : 3;
        CHECK(g_launches - before == 8 + 3 * step_launches + (fmt == VQKV_FMT_2BIT ? 1 : 2) + vt);
    }
    // Rejections: no launch may happen.
    const int before = g_launches;
    vqkv_shape bad = good;
    bad.head_dim = 64;
    CHECK(vqkv_decode_attention(&bad, Ff, Fb, Fb, Fc, Fc, 100, 0.088f, 1, F, nullptr) == VQKV_ERR_UNSUPPORTED);
    bad = good; bad.num_q_heads = 30;
    CHECK(vqkv_transform_query(&bad, F, 0, Ff, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    bad = good; bad.fmt = 5;
    CHECK(vqkv_cache_bytes(&bad) == 0);
    bad = good; bad.fmt = 0x200;
    CHECK(vqkv_quantize_append(&bad, F, F, 0, 1, 0, Ff, Fb, Fb, Fc, Fc, nullptr) == VQKV_ERR_INVALID_ARG);
    bad = good; bad.max_tokens = 100;
    CHECK(vqkv_decode_attention(&bad, Ff, Fb, Fb, Fc, Fc, 50, 0.088f, 1, F, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_attention(&good, Ff, Fb, Fb, Fc, Fc, 0, 0.088f, 1, F, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_attention(&good, Ff, Fb, Fb, Fc, Fc, 196609, 0.088f, 1, F, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_attention(&good, Ff, Fb, Fb, Fc, Fc, 100, NAN, 1, F, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_attention(&good, Ff, Fb, Fb, Fc, Fc, 100, 0.088f, 3, F, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_attention(&good, Ff, Fb, Fb, Fc, Fc, 100, 0.088f, 1, P(0x10004), nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_quantize_append(&good, F, F, 0, 0, 0, Ff, Fb, Fb, Fc, Fc, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_quantize_append(&good, F, F, 0, 2, 196607, Ff, Fb, Fb, Fc, Fc, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_quantize_append(&good, nullptr, F, 0, 1, 0, Ff, Fb, Fb, Fc, Fc, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_quantize_append(&good, F, F, 7, 1, 0, Ff, Fb, Fb, Fc, Fc, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_step(&good, F, F, F, 0, -1, Ff, Fb, Fb, Fc, Fc, 0.088f, 1, F, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_step(&good, F, F, F, 0, 196608, Ff, Fb, Fb, Fc, Fc, 0.088f, 1, F, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_step_paged(&good, F, F, F, 0, Fi, 100, Ff, Fb, Fb, Fc, Fc, 0, Fi, 0.088f, 1, F, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_step_varlen(&good, F, F, F, 0, nullptr, 100, Ff, Fb, Fb, Fc, Fc, 0.088f, 1, F, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_combine(&good, 0, F, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    // The allocation-free step: a workspace beyond the static scratch is refused.
    CHECK(vqkv_step_workspace_bytes(&good, 64) > VQKV_STATIC_SCRATCH_BYTES);
    CHECK(vqkv_decode_step_static(&good, F, F, F, 0, 196607, Ff, Fb, Fb, Fc, Fc, 0.088f, 64, Ff, nullptr) == VQKV_ERR_UNSUPPORTED);
    CHECK(vqkv_decode_step_static(&good, F, F, F, 0, 196607, Ff, Fb, Fb, Fc, Fc, 0.088f, 0, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_decode_step_static(&good, F, F, F, 0, -1, Ff, Fb, Fb, Fc, Fc, 0.088f, 1, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_train_codebook(1, 255, F, 0, 0, nullptr, static_cast<const int64_t*>(F), 20, static_cast<uint16_t*>(F), nullptr, F, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(vqkv_smooth_scales(0, 10, F, 0, Ff, nullptr) == VQKV_ERR_INVALID_ARG);
    CHECK(g_launches == before);
    CHECK(vqkv_status_string(VQKV_ERR_HIP)[0] != '\0' && vqkv_last_error()[0] != '\0');
    std::printf("abi driver ok\n");
    return 0;
}
