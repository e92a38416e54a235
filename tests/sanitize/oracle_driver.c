/* Drives every function of the oracle on small inputs, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (the test that builds it
 * treats any report or a failed self-check as a failure).  Test
 * infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int vqo_format(int fmt, int* entries, int* dsub);
double vqo_half_to_double(uint16_t h);
uint16_t vqo_double_to_half(double x);
void vqo_hadamard(double* H);
void vqo_fwht(double* x);
void vqo_smooth_scales(const double* k_cal, int64_t n, float* s);
void vqo_transform_key(const double* k, const float* s, double* out);
void vqo_transform_query(const double* q, const float* s, double* out);
void vqo_value_output_transform(double* o, const float* sv);
int vqo_nearest(const double* x, const double* book, int entries, int dsub);
int vqo_quantize(int fmt, int64_t n, const double* k, const double* v, const float* s, const float* sv,
                 const uint16_t* kbook16, const uint16_t* vbook16, uint16_t* kcodes, uint16_t* vcodes,
                 int nthreads);
void vqo_kmeans(int64_t n, int dsub, int E, const double* pts, const int64_t* init, int iters, double* cent,
                int32_t* assign, int nthreads);
int vqo_attention(int fmt, int B, int Hq, int Hkv, int64_t T, const double* q, const float* s, const float* sv,
                  const uint16_t* kbook16, const uint16_t* vbook16, const uint16_t* kcodes,
                  const uint16_t* vcodes, double sm_scale, double* out, int nthreads);
int vqo_attention_fp(int B, int Hq, int Hkv, int64_t T, const double* q, const double* k, const double* v,
                     double sm_scale, double* out, int nthreads);
int vqo_pack_k(int fmt, int64_t T, const uint16_t* codes, uint8_t* out);
int vqo_unpack_k(int fmt, int64_t T, const uint8_t* in, uint16_t* codes);
int vqo_pack_v(int fmt, int64_t T, const uint16_t* codes, uint8_t* out);
int vqo_unpack_v(int fmt, int64_t T, const uint8_t* in, uint16_t* codes);

#define HD 128
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {                    /* SplitMix64 -> [0, 1) */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1p-53;
}
static double nrand(void) { return sqrt(-2.0 * log(urand() + 1e-300)) * cos(6.283185307179586 * urand()); }

int main(void) {
    double H[HD * HD], x[HD], y[HD], z[HD];
    float s[HD], sv[HD];
    vqo_hadamard(H);
    for (int i = 0; i < HD; ++i) { x[i] = nrand(); s[i] = (float)(0.5 + 2.0 * urand()); sv[i] = (float)(0.5 + urand()); }
    memcpy(y, x, sizeof(x));
    vqo_fwht(y);
    vqo_fwht(y);                                              /* H H = I */
    for (int i = 0; i < HD; ++i) CHECK(fabs(y[i] - x[i]) < 1e-12);
    vqo_transform_key(x, sv, y);
    vqo_value_output_transform(y, sv);
    for (int i = 0; i < HD; ++i) CHECK(fabs(y[i] - x[i]) < 1e-12);
    vqo_transform_query(x, s, z);
    CHECK(vqo_double_to_half(vqo_half_to_double(0x3c00)) == 0x3c00);
    {
        double cal[64 * HD];
        for (int i = 0; i < 64 * HD; ++i) cal[i] = nrand();
        float sc[HD];
        vqo_smooth_scales(cal, 64, sc);
        for (int i = 0; i < HD; ++i) CHECK(sc[i] > 0.0f);
    }
    for (int fmt = 0; fmt < 5; ++fmt) {
        int E, dsub;
        CHECK(vqo_format(fmt, &E, &dsub) == 0);
        const int J = HD / dsub, n = 5, T = 70, cap = 128;
        const int W = fmt == 0 ? 32 : (fmt == 1 ? 24 : (fmt == 2 ? 48 : (fmt == 3 ? 20 : 64)));
        uint16_t* kb = malloc(sizeof(uint16_t) * E * dsub);
        uint16_t* vb = malloc(sizeof(uint16_t) * E * dsub);
        double* bookd = malloc(sizeof(double) * E * dsub);
        for (int i = 0; i < E * dsub; ++i) {
            kb[i] = vqo_double_to_half(0.6 * nrand());
            vb[i] = vqo_double_to_half(nrand());
            bookd[i] = vqo_half_to_double(kb[i]);
        }
        CHECK(vqo_nearest(x, bookd, E, dsub) >= 0);
        double k[5 * HD], v[5 * HD];
        for (int i = 0; i < n * HD; ++i) { k[i] = nrand(); v[i] = nrand(); }
        uint16_t kc[5 * 64], vc[5 * 64];
        CHECK(vqo_quantize(fmt, n, k, v, s, NULL, kb, vb, kc, vc, 2) == 0);
        CHECK(vqo_quantize(fmt, n, k, v, s, sv, kb, vb, kc, vc, 2) == 0);
        /* Codes of T tokens, packed and unpacked in both layouts. */
        uint16_t* codes = malloc(sizeof(uint16_t) * T * J);
        uint16_t* back = malloc(sizeof(uint16_t) * T * J);
        uint8_t* bytes = calloc((size_t)cap * W, 1);
        for (int i = 0; i < T * J; ++i) codes[i] = (uint16_t)(urand() * E);
        CHECK(vqo_pack_k(fmt, T, codes, bytes) == 0 && vqo_unpack_k(fmt, T, bytes, back) == 0);
        CHECK(memcmp(codes, back, sizeof(uint16_t) * T * J) == 0);
        CHECK(vqo_pack_v(fmt, T, codes, bytes) == 0 && vqo_unpack_v(fmt, T, bytes, back) == 0);
        CHECK(memcmp(codes, back, sizeof(uint16_t) * T * J) == 0);
        /* Attention: B 2, Hq 4, Hkv 2, T tokens; with and without the value map. */
        double q[2 * 4 * HD], out[2 * 4 * HD];
        float s2[2 * HD], sv2[2 * HD];
        for (int i = 0; i < 2 * 4 * HD; ++i) q[i] = nrand();
        for (int i = 0; i < 2 * HD; ++i) { s2[i] = s[i % HD]; sv2[i] = sv[i % HD]; }
        uint16_t* kb2 = malloc(sizeof(uint16_t) * 2 * E * dsub);
        uint16_t* vb2 = malloc(sizeof(uint16_t) * 2 * E * dsub);
        memcpy(kb2, kb, sizeof(uint16_t) * E * dsub); memcpy(kb2 + E * dsub, kb, sizeof(uint16_t) * E * dsub);
        memcpy(vb2, vb, sizeof(uint16_t) * E * dsub); memcpy(vb2 + E * dsub, vb, sizeof(uint16_t) * E * dsub);
        uint16_t* kcs = malloc(sizeof(uint16_t) * 2 * 2 * T * J);
        uint16_t* vcs = malloc(sizeof(uint16_t) * 2 * 2 * T * J);
        for (int i = 0; i < 4 * T * J; ++i) { kcs[i] = (uint16_t)(urand() * E); vcs[i] = (uint16_t)(urand() * E); }
        CHECK(vqo_attention(fmt, 2, 4, 2, T, q, s2, NULL, kb2, vb2, kcs, vcs, 0.0883883, out, 2) == 0);
        for (int i = 0; i < 2 * 4 * HD; ++i) CHECK(isfinite(out[i]));
        CHECK(vqo_attention(fmt, 2, 4, 2, T, q, s2, sv2, kb2, vb2, kcs, vcs, 0.0883883, out, 2) == 0);
        for (int i = 0; i < 2 * 4 * HD; ++i) CHECK(isfinite(out[i]));
        /* K-Means on the key book's entries as points. */
        const int npts = 2 * E;
        double* pts = malloc(sizeof(double) * npts * dsub);
        for (int i = 0; i < npts * dsub; ++i) pts[i] = nrand();
        int64_t* init = malloc(sizeof(int64_t) * E);
        for (int e = 0; e < E; ++e) init[e] = 2 * e;
        double* cent = malloc(sizeof(double) * E * dsub);
        int32_t* assign = malloc(sizeof(int32_t) * npts);
        vqo_kmeans(npts, dsub, E, pts, init, 2, cent, assign, 2);
        for (int i = 0; i < npts; ++i) CHECK(assign[i] >= 0 && assign[i] < E);
        free(kb); free(vb); free(bookd); free(codes); free(back); free(bytes); free(kb2); free(vb2);
        free(kcs); free(vcs); free(pts); free(init); free(cent); free(assign);
    }
    {
        double q[1 * 2 * HD], kk[1 * 1 * 9 * HD], vv[1 * 1 * 9 * HD], out[2 * HD];
        for (int i = 0; i < 2 * HD; ++i) q[i] = nrand();
        for (int i = 0; i < 9 * HD; ++i) { kk[i] = nrand(); vv[i] = nrand(); }
        CHECK(vqo_attention_fp(1, 2, 1, 9, q, kk, vv, 0.0883883, out, 2) == 0);
    }
    CHECK(vqo_format(7, &(int){0}, &(int){0}) != 0);
    printf("oracle driver ok\n");
    return 0;
}
