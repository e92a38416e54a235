/*
 * vqkv_oracle.c -- plain, slow, fp64 CPU oracle for decode attention over a
 * vector-quantized KV cache, as the VecInfer pages describe it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant generator with the HIP
 * path.
 *
 * Sources (page titles; no code is printed on any of them):
 *   [card]     "VecInfer: Efficient LLM Inference with Low-Bit KV Cache via
 *              Outlier-Suppressed Vector Quantization", research.elamur.ai
 *              summary card -- sections "Summary" and "Key points".
 *   [abstract] the same paper's arXiv 2510.06175 page (shd-paper.top):
 *              English abstract and the Chinese "technical framework" paragraph
 *              (three stages: preprocess keys, vector-quantize, fused kernel).
 *
 * What is computed (every function says which passage it follows):
 *   - smoothing scale per key channel, then a normalized Sylvester Hadamard
 *     rotation of the smoothed key; the query gets q*s and the same rotation,
 *     so q'.k' == q.k ([card] Summary; [abstract]);
 *   - nearest-centroid codes under squared L2 over contiguous sub-vectors,
 *     ties to the lowest index, with codebooks of 2^8 x 4 (2-bit) or
 *     2^12 x 8 (1.5-bit) fp16 entries ([card] Key points, codebook size),
 *     and two more widths inside the pages' 1.25-4 bit range ([card] Summary):
 *     2^12 x 4 (3-bit) and 2^10 x 8 (1.25-bit);
 *   - offline K-Means (Lloyd) codebooks ([card] Summary, "trained offline");
 *   - exact softmax attention over the dequantized cache, one query head at a
 *     time (the definition the fused kernel must reproduce; [abstract]).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - s_c = sqrt(max_t |Kcal[t][c]|), stored as the fp32 nearest the fp64 sqrt;
 *   - keys are divided by s before the rotation; values are not transformed,
 *     except in the value-transform variant (the technical-framework paragraph
 *     speaks of the preprocessed KV cache): values then get their own scales
 *     s_v and the same rotation, v' = H (v / s_v), and the attention output is
 *     mapped back, o = s_v * (H o'), since H is its own inverse;
 *   - the rotation is computed by the fast Walsh-Hadamard butterflies in stage
 *     order h = 1, 2, ..., 64, each (a, b) -> (a + b, a - b), then every element
 *     is multiplied by the fp64 nearest to 1/sqrt(128).  That pins the fp64
 *     rounding that decides codes; fwht() is checked against the explicit
 *     Sylvester matrix in the tests;
 *   - distance d_e = sum_i (x_i - c_e,i)^2, added left to right, no fused
 *     multiply-add (this file is built with -ffp-contract=off);
 *   - attention: q-head g reads KV head g / G; scores scaled by sm_scale;
 *     two-pass softmax.
 *
 * Code layouts in device memory (pack_k / pack_v) restate the library's
 * documented layout so tests can feed it and compare bytes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HD 128

/* fp64 nearest to 1/sqrt(128) = 2^-3.5; the tests check that this literal is
 * the correctly rounded value. */
static const double INV_SQRT_HD = 0x1.6a09e667f3bcdp-4;

int vqo_format(int fmt, int* entries, int* dsub)
{
    /* [card] Key points, codebook size: 2^8 entries x 4 dims for 2 bits,
     * 2^12 entries x 8 dims for 1.5 bits. */
    if (fmt == 0) { *entries = 256; *dsub = 4; return 0; }
    if (fmt == 1) { *entries = 4096; *dsub = 8; return 0; }
    /* A third bit-width inside the pages' 1.25-4 bit range (their results
     * span it; the shape is not printed): 2^12 entries x 4 dims, 3 bits per
     * element. */
    if (fmt == 2) { *entries = 4096; *dsub = 4; return 0; }
    /* The low end of that range, 1.25 bits per element ([card] Summary: the
     * results start at 1.25 bits; the shape is not printed): the 1.5-bit
     * setting's 8-dim sub-vectors with 2^10 entries, 10-bit codes. */
    if (fmt == 3) { *entries = 1024; *dsub = 8; return 0; }
    /* The high end, 4 bits per element: 2^8 entries x 2 dims (8-bit codes on
     * 2-dim sub-vectors; the shape is not printed either). */
    if (fmt == 4) { *entries = 256; *dsub = 2; return 0; }
    return -1;
}

/* Bytes of one token's codes per (b, KV head): 32 (2-bit), 24 (1.5-bit),
 * 48 (3-bit), 20 (1.25-bit), 64 (4-bit). */
static int code_bytes(int fmt)
{
    switch (fmt) {
    case 0: return 32;
    case 1: return 24;
    case 2: return 48;
    case 3: return 20;
    default: return 64;
    }
}

/* ------------------------------------------------------------------ fp16 */

/* IEEE 754 binary16 -> double, from the format's definition. */
double vqo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);                 /* subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), exp - 25);  /* (1024 + man) * 2^(exp-25) */
    return sign ? -v : v;
}

/* double -> binary16, round to nearest, ties to even; overflow to infinity. */
uint16_t vqo_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    if (a == 0.0) return sign;
    /* Largest finite half is 65504; values at or above 65520 round to infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    int e;
    frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
    int unbiased = e - 1;         /* a in [2^unbiased, 2^(unbiased+1)) */
    double quantum;               /* spacing of halves around a */
    if (unbiased < -14) quantum = ldexp(1.0, -24);        /* subnormal range */
    else quantum = ldexp(1.0, unbiased - 10);
    double q = a / quantum;       /* exact: quantum is a power of two */
    double fl = floor(q);
    double rem = q - fl;
    double n = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    double r = n * quantum;       /* the rounded magnitude, exactly representable */
    /* Encode r. */
    if (r < ldexp(1.0, -14)) {
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    }
    if (r >= 65520.0) return (uint16_t)(sign | 0x7c00);
    int re;
    double rf = frexp(r, &re);    /* r = rf * 2^re */
    int hexp = re - 1 + 15;
    int man = (int)(ldexp(rf, 11) - 1024.0);
    return (uint16_t)(sign | (hexp << 10) | man);
}

/* ------------------------------------------------------------ transforms */

/* The normalized Sylvester Hadamard matrix of order 128 by its definition:
 * H[i][j] = (-1)^popcount(i & j) / sqrt(128). */
void vqo_hadamard(double* H)
{
    for (int i = 0; i < HD; ++i)
        for (int j = 0; j < HD; ++j) {
            int bits = __builtin_popcount((unsigned)(i & j));
            H[i * HD + j] = (bits & 1) ? -INV_SQRT_HD : INV_SQRT_HD;
        }
}

/* y = H x by the fast Walsh-Hadamard butterflies, in the pinned stage order. */
void vqo_fwht(double* x)
{
    for (int h = 1; h < HD; h <<= 1)
        for (int i = 0; i < HD; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
    for (int i = 0; i < HD; ++i) x[i] = x[i] * INV_SQRT_HD;
}

/* [card] Summary: channel-wise smoothing of the keys.  Reading: per channel c,
 * s_c = sqrt(max_t |k_cal[t][c]|), stored as fp32 (the fp32 nearest the fp64
 * square root).  k_cal is [n][128]. */
void vqo_smooth_scales(const double* k_cal, int64_t n, float* s)
{
    for (int c = 0; c < HD; ++c) {
        double m = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            double a = fabs(k_cal[t * HD + c]);
            if (a > m) m = a;
        }
        s[c] = (float)sqrt(m);
    }
}

/* [card] Summary: smooth, then rotate.  x' = H (k / s). */
void vqo_transform_key(const double* k, const float* s, double* out)
{
    for (int i = 0; i < HD; ++i) out[i] = k[i] / (double)s[i];
    vqo_fwht(out);
}

/* [card] Summary: the matching inverse on the query keeps q'.k' = q.k:
 * (H (k/s)) . (H (q*s)) = (k/s) . (q*s) = k . q, H being symmetric orthogonal. */
void vqo_transform_query(const double* q, const float* s, double* out)
{
    for (int i = 0; i < HD; ++i) out[i] = q[i] * (double)s[i];
    vqo_fwht(out);
}

/* Value-transform variant: the inverse of v' = H (v / s_v) applied to an
 * attention output, o = s_v * (H o').  In place on o[128]. */
void vqo_value_output_transform(double* o, const float* sv)
{
    vqo_fwht(o);
    for (int i = 0; i < HD; ++i) o[i] = o[i] * (double)sv[i];
}

/* ------------------------------------------------------- nearest centroid */

/* Index of the nearest centroid of `book` ([entries][dsub], fp64) to x[dsub]
 * under squared L2, lowest index among equals. */
int vqo_nearest(const double* x, const double* book, int entries, int dsub)
{
    double best = INFINITY;
    int idx = 0;
    for (int e = 0; e < entries; ++e) {
        const double* c = book + (int64_t)e * dsub;
        double t = x[0] - c[0];
        double d = t * t;
        for (int i = 1; i < dsub; ++i) {
            t = x[i] - c[i];
            d = d + t * t;
        }
        if (d < best) { best = d; idx = e; }
    }
    return idx;
}

static double* decode_book(const uint16_t* book16, int entries, int dsub)
{
    double* b = (double*)malloc(sizeof(double) * (size_t)entries * dsub);
    for (int64_t i = 0; i < (int64_t)entries * dsub; ++i) b[i] = vqo_half_to_double(book16[i]);
    return b;
}

/* [abstract] stages 1-2: transform new keys, then vector-quantize keys and
 * values.  k, v: [n][128] fp64 values; s: [128]; sv: [128] or NULL (values
 * untransformed); books fp16 [E][dsub].
 * Codes out: [n][J] with J = 128 / dsub; sub-vector j covers dims
 * [j*dsub, (j+1)*dsub). */
int vqo_quantize(int fmt, int64_t n, const double* k, const double* v, const float* s,
                 const float* sv, const uint16_t* kbook16, const uint16_t* vbook16,
                 uint16_t* kcodes, uint16_t* vcodes, int nthreads)
{
    int E, dsub;
    if (vqo_format(fmt, &E, &dsub)) return -1;
    int J = HD / dsub;
    double* kb = decode_book(kbook16, E, dsub);
    double* vb = decode_book(vbook16, E, dsub);
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double x[HD], xv[HD];
        vqo_transform_key(k + t * HD, s, x);
        /* Value-transform variant (sv non-NULL): the values get the keys' steps
         * with their own scales. */
        const double* vt = v + t * HD;
        if (sv) {
            vqo_transform_key(vt, sv, xv);
            vt = xv;
        }
        for (int j = 0; j < J; ++j) {
            kcodes[t * J + j] = (uint16_t)vqo_nearest(x + j * dsub, kb, E, dsub);
            vcodes[t * J + j] = (uint16_t)vqo_nearest(vt + j * dsub, vb, E, dsub);
        }
    }
    free(kb);
    free(vb);
    return 0;
}

/* ---------------------------------------------------------------- K-Means */

/* [card] Summary: a K-Means codebook trained offline.  Lloyd's iterations
 * from given initial points (indices into pts): assign each point to the
 * nearest centroid (rule of vqo_nearest), then move every centroid to the mean
 * of its points (summed in point order); a centroid with no points stays.
 * pts: [n][dsub].  Outputs fp64 centroids [E][dsub] and the last assignment. */
void vqo_kmeans(int64_t n, int dsub, int E, const double* pts, const int64_t* init,
                int iters, double* cent, int32_t* assign, int nthreads)
{
    for (int e = 0; e < E; ++e)
        for (int i = 0; i < dsub; ++i) cent[(int64_t)e * dsub + i] = pts[init[e] * dsub + i];
    double* sums = (double*)malloc(sizeof(double) * (size_t)E * dsub);
    int64_t* counts = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
    for (int it = 0; it < iters; ++it) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int64_t p = 0; p < n; ++p) assign[p] = vqo_nearest(pts + p * dsub, cent, E, dsub);
        memset(sums, 0, sizeof(double) * (size_t)E * dsub);
        memset(counts, 0, sizeof(int64_t) * (size_t)E);
        for (int64_t p = 0; p < n; ++p) {
            int a = assign[p];
            counts[a] += 1;
            for (int i = 0; i < dsub; ++i) sums[(int64_t)a * dsub + i] += pts[p * dsub + i];
        }
        for (int e = 0; e < E; ++e)
            if (counts[e] > 0)
                for (int i = 0; i < dsub; ++i)
                    cent[(int64_t)e * dsub + i] = sums[(int64_t)e * dsub + i] / (double)counts[e];
    }
    free(sums);
    free(counts);
}

/* -------------------------------------------------------------- attention */

/* Exact decode attention over the dequantized cache ([abstract]: the kernel
 * fuses dequantization into attention; this is the result it must reach).
 *   q      [B][Hq][128]        query values
 *   s      [Hkv][128]          smoothing scales
 *   books  [Hkv][E][dsub]      fp16
 *   codes  [B][Hkv][T][J]      indices
 *   out    [B][Hq][128]
 * For q-head g of KV head h = g / (Hq/Hkv):
 *   q' = H (q * s_h);  z_t = sm_scale * sum_j q'_j-slice . C_K[kc_t,j];
 *   p = exp(z - max z) / sum;  o = sum_t p_t * concat_j C_V[vc_t,j]. */
int vqo_attention(int fmt, int B, int Hq, int Hkv, int64_t T, const double* q, const float* s,
                  const float* sv, const uint16_t* kbook16, const uint16_t* vbook16,
                  const uint16_t* kcodes, const uint16_t* vcodes, double sm_scale,
                  double* out, int nthreads)
{
    int E, dsub;
    if (vqo_format(fmt, &E, &dsub)) return -1;
    if (Hkv <= 0 || Hq % Hkv != 0 || T < 1) return -1;
    int J = HD / dsub, G = Hq / Hkv;
    double* kb = decode_book(kbook16, E, dsub * Hkv);
    double* vb = decode_book(vbook16, E, dsub * Hkv);
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t bg = 0; bg < (int64_t)B * Hq; ++bg) {
        int b = (int)(bg / Hq), g = (int)(bg % Hq), h = g / G;
        double qp[HD];
        vqo_transform_query(q + bg * HD, s + (int64_t)h * HD, qp);
        const double* kbh = kb + (int64_t)h * E * dsub;
        const double* vbh = vb + (int64_t)h * E * dsub;
        const uint16_t* kc = kcodes + ((int64_t)b * Hkv + h) * T * J;
        const uint16_t* vc = vcodes + ((int64_t)b * Hkv + h) * T * J;
        double* z = (double*)malloc(sizeof(double) * (size_t)T);
        double m = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int j = 0; j < J; ++j) {
                const double* c = kbh + (int64_t)kc[t * J + j] * dsub;
                for (int i = 0; i < dsub; ++i) acc += qp[j * dsub + i] * c[i];
            }
            z[t] = sm_scale * acc;
            if (z[t] > m) m = z[t];
        }
        double l = 0.0, o[HD];
        for (int d = 0; d < HD; ++d) o[d] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double w = exp(z[t] - m);
            l += w;
            for (int j = 0; j < J; ++j) {
                const double* c = vbh + (int64_t)vc[t * J + j] * dsub;
                for (int i = 0; i < dsub; ++i) o[j * dsub + i] += w * c[i];
            }
        }
        for (int d = 0; d < HD; ++d) o[d] = o[d] / l;
        /* Value-transform variant: the output of the rotated values mapped back. */
        if (sv) vqo_value_output_transform(o, sv + (int64_t)h * HD);
        for (int d = 0; d < HD; ++d) out[bg * HD + d] = o[d];
        free(z);
    }
    free(kb);
    free(vb);
    return 0;
}

/* Full-precision attention on raw keys and values (quality reference and the
 * invariance pins): out = softmax(sm_scale * q.k) v.  k, v: [B][Hkv][T][128]. */
int vqo_attention_fp(int B, int Hq, int Hkv, int64_t T, const double* q, const double* k,
                     const double* v, double sm_scale, double* out, int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || T < 1) return -1;
    int G = Hq / Hkv;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t bg = 0; bg < (int64_t)B * Hq; ++bg) {
        int b = (int)(bg / Hq), g = (int)(bg % Hq), h = g / G;
        const double* kk = k + ((int64_t)b * Hkv + h) * T * HD;
        const double* vv = v + ((int64_t)b * Hkv + h) * T * HD;
        const double* qq = q + bg * HD;
        double* z = (double*)malloc(sizeof(double) * (size_t)T);
        double m = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int d = 0; d < HD; ++d) acc += qq[d] * kk[t * HD + d];
            z[t] = sm_scale * acc;
            if (z[t] > m) m = z[t];
        }
        double l = 0.0, o[HD];
        for (int d = 0; d < HD; ++d) o[d] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double w = exp(z[t] - m);
            l += w;
            for (int d = 0; d < HD; ++d) o[d] += w * vv[t * HD + d];
        }
        for (int d = 0; d < HD; ++d) out[bg * HD + d] = o[d] / l;
        free(z);
    }
    return 0;
}

/* ---------------------------------------------------------------- layouts */

/* The library's code layout for one (batch, KV head) stream of capacity
 * `cap` tokens (a multiple of 64), restated from its header:
 *
 * Keys, token-major: token t occupies bytes [t*W, (t+1)*W), W = 32 (2-bit),
 * 24 (1.5-bit), 48 (3-bit), 20 (1.25-bit: 10-bit codes as bit fields, see
 * put_bits below) or 64 (4-bit).  2-bit and 4-bit: byte j = code of sub-vector j.  1.5-bit: sub-vectors
 * (2i, 2i+1) share bytes 3i..3i+2 as b0 = c0 & 0xFF, b1 = (c0 >> 8) | ((c1 & 0xF) << 4),
 * b2 = c1 >> 4 (12-bit codes, 3 bytes per 2 sub-vectors).
 *
 * Values, in blocks of 64 tokens (see v_offset): 2-bit blocks of 2048 bytes
 * (64 chunks of 32 bytes), 1.5-bit blocks of 1536 bytes (32 streams of 48
 * bytes, each holding 16 pairs of 12-bit codes by the same rule; a pair is
 * sub-vectors j and j + 8 of one token).
 *
 * codes: [T][J]; out: cap * W bytes.  Bytes of tokens >= T are left as they are. */
static void put12(uint8_t* p, int which, uint16_t c)
{
    if (which == 0) {
        p[0] = (uint8_t)(c & 0xff);
        p[1] = (uint8_t)((p[1] & 0xf0) | ((c >> 8) & 0x0f));
    } else {
        p[1] = (uint8_t)((p[1] & 0x0f) | ((c & 0x0f) << 4));
        p[2] = (uint8_t)((c >> 4) & 0xff);
    }
}

static uint16_t get12(const uint8_t* p, int which)
{
    if (which == 0) return (uint16_t)(p[0] | ((p[1] & 0x0f) << 8));
    return (uint16_t)((p[1] >> 4) | (p[2] << 4));
}

/* 10-bit codes (1.25-bit format) as little-endian bit fields: bit i of the
 * field is bit (pos + i) % 8 of byte (pos + i) / 8, one bit at a time.  Four
 * codes fill five bytes; the 12-bit pair rule above is the same convention. */
static void put_bits(uint8_t* p, int64_t pos, int width, uint32_t v)
{
    for (int i = 0; i < width; ++i) {
        int64_t b = pos + i;
        uint8_t m = (uint8_t)(1u << (b % 8));
        if ((v >> i) & 1u) p[b / 8] = (uint8_t)(p[b / 8] | m);
        else p[b / 8] = (uint8_t)(p[b / 8] & ~m);
    }
}

static uint32_t get_bits(const uint8_t* p, int64_t pos, int width)
{
    uint32_t v = 0;
    for (int i = 0; i < width; ++i) {
        int64_t b = pos + i;
        v |= (uint32_t)((p[b / 8] >> (b % 8)) & 1u) << i;
    }
    return v;
}

/* Keys of the 1.25-bit format: token-major, 20 bytes per token, the code of
 * sub-vector j in bits [10 j, 10 j + 10) of the token's bytes. */
int vqo_pack_k(int fmt, int64_t T, const uint16_t* codes, uint8_t* out)
{
    int E, dsub;
    if (vqo_format(fmt, &E, &dsub)) return -1;
    int J = HD / dsub;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < J; ++j) {
            uint16_t c = codes[t * J + j];
            if (fmt == 0 || fmt == 4) out[t * code_bytes(fmt) + j] = (uint8_t)c;
            else if (fmt == 3) put_bits(out + t * 20, 10 * j, 10, c);
            else put12(out + t * code_bytes(fmt) + 3 * (j / 2), j & 1, c);
        }
    return 0;
}

int vqo_unpack_k(int fmt, int64_t T, const uint8_t* in, uint16_t* codes)
{
    int E, dsub;
    if (vqo_format(fmt, &E, &dsub)) return -1;
    int J = HD / dsub;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < J; ++j) {
            if (fmt == 0 || fmt == 4) codes[t * J + j] = in[t * code_bytes(fmt) + j];
            else if (fmt == 3) codes[t * J + j] = (uint16_t)get_bits(in + t * 20, 10 * j, 10);
            else codes[t * J + j] = get12(in + t * code_bytes(fmt) + 3 * (j / 2), j & 1);
        }
    return 0;
}

/* Values of the 1.25-bit format: 64-token blocks of 1280 bytes, 32 streams of
 * 40 bytes.  As in the 1.5-bit layout, stream 8*((j%8)/2) + 2*(u%4) + j%2
 * (u = t % 64) holds the pairs (sub-vector j%8, sub-vector j%8 + 8) of the
 * tokens with that u % 4, pair u/4 in bits [20 (u/4), 20 (u/4) + 20) of the
 * stream's bytes, sub-vector j in the pair's 10-bit half j / 8.  Returns the
 * bit position of (t, j) from the start of the cache. */
static int64_t v_bit_1p25(int64_t t, int j)
{
    int64_t u = t % 64;
    int64_t stream = 8 * ((j % 8) / 2) + 2 * (u % 4) + (j % 2);
    return ((t / 64) * 1280 + 40 * stream) * 8 + 20 * (u / 4) + 10 * (j / 8);
}

static int64_t v_offset(int fmt, int64_t t, int j, int* which)
{
    if (fmt == 0) {
        /* 64-token blocks of 2048 bytes, 64 chunks of 32 bytes.  Chunk
           16*((j%16)/4) + 4*(u%4) + j%4 (u = t % 64) holds, at byte
           2*(u/4) + j/16, the code of sub-vector j of token t. */
        int64_t u = t % 64;
        int64_t chunk = 16 * ((j % 16) / 4) + 4 * (u % 4) + (j % 4);
        *which = 0;
        return (t / 64) * 2048 + 32 * chunk + 2 * (u / 4) + j / 16;
    }
    if (fmt == 4) {
        /* 64-token blocks of 4096 bytes, 64 chunks of 64 bytes.  Sub-vectors
           2w and 2w+1 (4 dims) are group w of the 2-bit layout's 32: chunk
           16*((w%16)/4) + 4*(u%4) + w%4 (u = t % 64, w = j / 2) holds, at byte
           4*(u/4) + 2*(w/16) + j%2, the code of sub-vector j of token t. */
        int64_t u = t % 64;
        int w = j / 2;
        int64_t chunk = 16 * ((w % 16) / 4) + 4 * (u % 4) + (w % 4);
        *which = 0;
        return (t / 64) * 4096 + 64 * chunk + 4 * (u / 4) + 2 * (w / 16) + (j % 2);
    }
    if (fmt == 2) {
        /* 64-token blocks of 3072 bytes, 64 chunks of 48 bytes.  Chunk
           16*((j%16)/4) + 4*(u%4) + j%4 (u = t % 64, as in the 2-bit layout)
           holds, in bytes 3*(u/4)..3*(u/4)+2, the pair (sub-vector j%16,
           sub-vector j%16 + 16) of token t; sub-vector j is element j/16. */
        int64_t u = t % 64;
        int64_t chunk = 16 * ((j % 16) / 4) + 4 * (u % 4) + (j % 4);
        *which = j / 16;
        return (t / 64) * 3072 + 48 * chunk + 3 * (u / 4);
    }
    {
        /* 64-token blocks of 1536 bytes, 32 streams of 48 bytes.  Stream
           8*((j%8)/2) + 2*(u%4) + j%2 (u = t % 64) holds, in bytes
           3*(u/4)..3*(u/4)+2, the pair (sub-vector j%8, sub-vector j%8 + 8)
           of token t; sub-vector j is element j/8 of the pair. */
        int64_t u = t % 64;
        int64_t stream = 8 * ((j % 8) / 2) + 2 * (u % 4) + (j % 2);
        *which = j / 8;
        return (t / 64) * 1536 + 48 * stream + 3 * (u / 4);
    }
}

int vqo_pack_v(int fmt, int64_t T, const uint16_t* codes, uint8_t* out)
{
    int E, dsub;
    if (vqo_format(fmt, &E, &dsub)) return -1;
    int J = HD / dsub;
    if (fmt == 3) {
        for (int64_t t = 0; t < T; ++t)
            for (int j = 0; j < J; ++j) put_bits(out, v_bit_1p25(t, j), 10, codes[t * J + j]);
        return 0;
    }
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < J; ++j) {
            int which;
            int64_t off = v_offset(fmt, t, j, &which);
            if (fmt == 0 || fmt == 4) out[off] = (uint8_t)codes[t * J + j];
            else put12(out + off, which, codes[t * J + j]);
        }
    return 0;
}

int vqo_unpack_v(int fmt, int64_t T, const uint8_t* in, uint16_t* codes)
{
    int E, dsub;
    if (vqo_format(fmt, &E, &dsub)) return -1;
    int J = HD / dsub;
    if (fmt == 3) {
        for (int64_t t = 0; t < T; ++t)
            for (int j = 0; j < J; ++j) codes[t * J + j] = (uint16_t)get_bits(in, v_bit_1p25(t, j), 10);
        return 0;
    }
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < J; ++j) {
            int which;
            int64_t off = v_offset(fmt, t, j, &which);
            codes[t * J + j] = (fmt == 0 || fmt == 4) ? in[off] : get12(in + off, which);
        }
    return 0;
}
