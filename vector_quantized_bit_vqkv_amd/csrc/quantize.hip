// quantize.hip -- key/value quantization into codebook indices, and the offline
// calibration that produces the smoothing scales and K-Means codebooks.
//
// VecInfer summary card, "Summary", and the arXiv 2510.06175 page's
// "technical framework" paragraph: keys are smoothed per channel and rotated
// by a Hadamard transform, then keys and values are vector-quantized against
// codebooks trained offline with K-Means ("Key points": 2^8 x 4 entries for
// 2-bit, 2^12 x 8 for 1.5-bit; two more widths inside the pages' 1.25-4 bit
// range, 2^12 x 4 at 3 bits and 2^10 x 8 at 1.25 bits, take the same steps).  In the value-transform
// variant the values take the keys' steps with their own scales s_v.
//
// Every decision that turns floating point into an integer (a code, a K-Means
// assignment) is taken in fp64 with one fixed operation sequence, so the
// result is exactly reproducible:
//   x = k / s            (fp64 divide, correctly rounded)
//   FWHT butterflies     stage h = 1, 2, ..., 64, pair (j, j + h) -> (a + b, a - b)
//   x *= 0x1.6a09e667f3bcdp-4   (fp64 nearest 1/sqrt(128))
//   d_e = (x0 - c0)^2 + (x1 - c1)^2 + ...   left to right, no fused multiply-add
//   code = the lowest e with the smallest d_e
// This file is compiled with -ffp-contract=off and also says so below.
#include "device_util.h"
#include "internal.h"
#include "qtransform.h"
#include "token_search.h"

#pragma clang fp contract(off)

namespace vqkv {

namespace {

template <int FMT> struct Fmt;
template <> struct Fmt<0> { static constexpr int E = 256, DS = 4, J = 32, W = 32; };
template <> struct Fmt<1> { static constexpr int E = 4096, DS = 8, J = 16, W = 24; };
template <> struct Fmt<2> { static constexpr int E = 4096, DS = 4, J = 32, W = 48; };
template <> struct Fmt<3> { static constexpr int E = 1024, DS = 8, J = 16, W = 20; };
template <> struct Fmt<4> { static constexpr int E = 256, DS = 2, J = 64, W = 64; };

// Writes the `width`-bit field v (width <= 56) at bit `bit` of the little-endian
// byte string p, keeping every bit outside the field (1.25-bit codes: 10-bit
// fields that do not start on byte boundaries).
__device__ __forceinline__ void put_field(uint8_t* p, int64_t bit, int width, uint64_t v) {
    uint8_t* q = p + (bit >> 3);
    const int sh = (int)(bit & 7), nb = (sh + width + 7) >> 3;
    uint64_t w = 0;
    for (int i = 0; i < nb; ++i) w |= (uint64_t)q[i] << (8 * i);
    const uint64_t mask = ((1ull << width) - 1ull) << sh;
    w = (w & ~mask) | ((v << sh) & mask);
    for (int i = 0; i < nb; ++i) q[i] = (uint8_t)(w >> (8 * i));
}

// 1.25-bit keys: the token's four 10-bit codes c[0..3] of sub-vectors 4i..4i+3
// fill bytes 5i..5i+4 of its 20 bytes.
__device__ __forceinline__ void put_key_group_1p25(uint8_t* tok, int i, const uint16_t* c) {
    const uint64_t v = (uint64_t)c[0] | ((uint64_t)c[1] << 10) | ((uint64_t)c[2] << 20) | ((uint64_t)c[3] << 30);
    put_field(tok, 40 * i, 40, v);
}

// Byte offset of the value pair (j, j + J/2) of token t, 12-bit formats.
template <int FMT>
__device__ __forceinline__ int64_t v_pair_offset(int64_t t, int j) {
    return FMT == 1 ? v_pair_offset_1p5(t, j) : v_pair_offset_3bit(t, j);
}

// In-place normalized FWHT of `ntok` rows of 128 fp64 values in LDS, by the
// whole block.  Caller synchronizes before (data written) and after.
__device__ void block_fwht(double* x, int ntok) {
    const int nb = ntok * 64;   // butterflies per stage
    for (int h = 1; h < kHeadDim; h <<= 1) {
        for (int idx = threadIdx.x; idx < nb; idx += blockDim.x) {
            const int tok = idx >> 6, pr = idx & 63;
            const int i = (pr / h) * 2 * h + (pr % h);
            double* r = x + tok * kHeadDim;
            const double a = r[i], b = r[i + h];
            r[i] = a + b;
            r[i + h] = a - b;
        }
        __syncthreads();
    }
    for (int idx = threadIdx.x; idx < ntok * kHeadDim; idx += blockDim.x) x[idx] = x[idx] * kInvSqrtHeadDimD;
    __syncthreads();
}

// Nearest entry among [e0, e1) of a book in LDS, widened to fp64 once when
// staged (the conversions were a fifth of the scan's instructions); strict
// "<" keeps the lowest index.
template <int DS>
__device__ __forceinline__ void argmin_range(const double* x, const double* book, int e0, int e1,
                                             double& best, int& idx) {
    best = __builtin_inf();
    idx = e0;
    for (int e = e0; e < e1; ++e) {
        const double d = dist_f64<DS>(x, book + e * DS);
        if (d < best) { best = d; idx = e; }
    }
}

// ------------------------------------------------- matrix-core distance screen
//
// Nearest centroid by a screen and an exact refinement, a set of points at a time:
// s~_e = |c_e|^2 - 2 x.c_e on v_mfma_f32_4x4x4f16, with x split into fp16
// hi + lo parts (each rounded through fp32: two hardware conversions instead
// of a software double-to-half rounding; products exact, fp32 sums) and
// broadcast to all 16 blocks (CBSZ = 4, ABID = group of 4 points), each lane
// holding one centroid of a 64-centroid group.  |s~_e - s_e| <= tau, with
// s_e = |c_e|^2 - 2 x.c_e exact
// and tau = 2^-18 (|x| + max|c|)^2 + 2^-22 max|c|_1 (twice the worst case of
// the x split, 18 fp32 accumulations, the fp32 |c|^2 and the final rounding).
// Every centroid with s~ <= min s~ + 3 tau is a candidate; candidates get the
// exact fp64 distance in the pinned order and the lowest index among the
// smallest wins, so the code equals the brute-force one.  Each lane keeps its
// best and second-best screened value (updated with selects, not branches:
// the screen is bound by VALU issue): when a lane's second value is also a
// candidate, or a coordinate is outside the fp16 range (|x| >= 2^15, NaN),
// the point falls back to the exact scan of the whole book.

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// x = hi + lo + err, both parts rounded through fp32 with the hardware
// conversions: |x - hi| <= 2^-11 (1 + 2^-12) |x|, |err| <= 2^-22 (1 + 2^-10) |x|
// + 2^-25 (lo subnormal), inside the bound's margin for the x split.
__device__ __forceinline__ _Float16 split_hi(double v) { return (_Float16)(float)v; }
__device__ __forceinline__ _Float16 split_lo(double v, _Float16 hi) { return (_Float16)(float)(v - (double)hi); }

template <int V> struct IntC { static constexpr int value = V; };
template <int I, int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    if constexpr (I < N) {
        f(IntC<I>{});
        static_for<I + 1, N>(f);
    }
}

template <int ABID>
__device__ __forceinline__ float4_t mfma_bcast(half4_t a, half4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}

// Lexicographic (distance, index) minimum over the wave; every lane gets it.
__device__ __forceinline__ void wave_argmin(double& d, int& idx) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const double od = __shfl_xor(d, m, 64);
        const int oi = __shfl_xor(idx, m, 64);
        if (od < d || (od == d && oi < idx)) { d = od; idx = oi; }
    }
}

__device__ __forceinline__ float wave_minf(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = fminf(v, __shfl_xor(v, m, 64));
    return v;
}

// Per-book constants of the bound, and |c_e|^2 in fp32 (exact products,
// DS - 1 additions): written by the whole block.
template <int DS, int E>
__device__ void book_norms(const uint16_t* book, float* cc, float* cmax2) {
    __shared__ float red[2][32];
    float m2 = 0.0f, m1 = 0.0f;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        float n2 = 0.0f, n1 = 0.0f;
#pragma unroll
        for (int i = 0; i < DS; ++i) {
            const float c = half_bits_to_float(book[e * DS + i]);
            n2 = n2 + c * c;
            n1 = n1 + fabsf(c);
        }
        cc[e] = n2;
        m2 = fmaxf(m2, n2);
        m1 = fmaxf(m1, n1);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        m2 = fmaxf(m2, __shfl_xor(m2, m, 64));
        m1 = fmaxf(m1, __shfl_xor(m1, m, 64));
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { red[0][w] = m2; red[1][w] = m1; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float a2 = 0.0f, a1 = 0.0f;
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) { a2 = fmaxf(a2, red[0][i]); a1 = fmaxf(a1, red[1][i]); }
        // fp32 rounding of the norms is far inside the bound's margin; round up anyway.
        cmax2[0] = a2 * (1.0f + 0x1p-20f);
        cmax2[1] = a1 * (1.0f + 0x1p-20f);
    }
    __syncthreads();
}

// The screen for one wave's set of 4 * NG points (A operands in lanes
// 0 .. 4 NG - 1: lane p holds point p) over centroid groups cg = cg0,
// cg0 + cgs, ...; per lane and point: best value m1 at centroid a1 (first
// index on ties), second value m2.
template <int DS, int E, int NG>
__device__ __forceinline__ void screen_set(const half4_t (&ahi)[DS / 4], const half4_t (&alo)[DS / 4],
                                           const uint16_t* book, const float* cc, int cg0, int cgs,
                                           float (&m1)[4 * NG], float (&m2)[4 * NG], int (&a1)[4 * NG]) {
    const int lane = threadIdx.x & 63;
#pragma unroll 1
    for (int cg = cg0; cg < E / 64; cg += cgs) {
        const int e = cg * 64 + lane;
        half4_t bq[DS / 4];
#pragma unroll
        for (int q = 0; q < DS / 4; ++q) bq[q] = *(const half4_t*)(book + e * DS + 4 * q);
        const float c2 = cc[e];
        static_for<0, NG>([&](auto gc) {
            constexpr int g = decltype(gc)::value;
            float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int q = 0; q < DS / 4; ++q) {
                d = mfma_bcast<g>(ahi[q], bq[q], d);
                d = mfma_bcast<g>(alo[q], bq[q], d);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pt = 4 * g + i;
                const float v = __builtin_fmaf(-2.0f, d[i], c2);
                const bool lt1 = v < m1[pt], lt2 = v < m2[pt];
                m2[pt] = lt1 ? m1[pt] : (lt2 ? v : m2[pt]);
                a1[pt] = lt1 ? e : a1[pt];
                m1[pt] = lt1 ? v : m1[pt];
            }
        });
    }
}

// Builds the A operands of up to NP points (point p of x, DS doubles each,
// for p < np) in lanes 0 .. NP - 1; flags points outside the fp16 range;
// returns |x| of point (lane % NP).
template <int DS, int NP>
__device__ __forceinline__ double screen_operands(const double* x, int np, half4_t (&ahi)[DS / 4],
                                                  half4_t (&alo)[DS / 4], bool& out_of_range) {
    const int p = threadIdx.x & (NP - 1);
    double n2 = 0.0;
    out_of_range = false;
#pragma unroll
    for (int q = 0; q < DS / 4; ++q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double v = p < np ? x[p * DS + 4 * q + i] : 0.0;
            n2 = n2 + v * v;
            if (!(__builtin_fabs(v) < 32768.0)) out_of_range = true;
            ahi[q][i] = split_hi(v);
            alo[q][i] = split_lo(v, ahi[q][i]);
        }
    }
    return __builtin_sqrt(n2);
}

// -------------------------------------------------------------- append kernel

// Tiles are TT-aligned; 1.25-bit value pairs of tokens u, u + 4 (u % 8 < 4) share
// bytes, so its tiles must hold whole 8-token groups (TT a multiple of 8).
template <int FMT> struct AppendTile { static constexpr int TT = (FMT == 0 || FMT == 4) ? 32 : 16; };   // 12-, 10-bit: 16

// The screen's bound for a point of norm xn against a book with
// (max |c|^2, max |c|_1) = cb.
__device__ __forceinline__ double screen_tau(double xn, const float* cb) {
    const double r = xn + __builtin_sqrt((double)cb[0]);
    return 0x1p-18 * r * r + 0x1p-22 * (double)cb[1];
}

// Final code of point p of a wave's screened set (see the screen): the
// candidates' exact distances, or the exact scan of the book on fallback.
template <int DS, int E>
__device__ __forceinline__ int refine_point(const double* xp, const uint16_t* book, double thr, bool fallback,
                                            float m1, int a1) {
    const int lane = threadIdx.x & 63;
    double d;
    int idx;
    if (!fallback) {
        const bool cand = (double)m1 <= thr;
        d = cand ? dist_h<DS>(xp, book + a1 * DS) : __builtin_inf();
        idx = cand ? a1 : 0x7fffffff;
    } else {
        d = __builtin_inf();
        idx = lane;                                   // lowest index when nothing compares smaller
        for (int e = lane; e < E; e += 64) {
            const double dd = dist_h<DS>(xp, book + e * DS);
            if (dd < d) { d = dd; idx = e; }
        }
    }
    wave_argmin(d, idx);
    return idx;
}

// Writes the 1.25-bit codes of tile rows [off, off + nt) (positions
// tile_base + row; kcodes / vcodes [TT][16]): keys in whole 5-byte groups of
// their token; values per 5-byte group of a stream, which holds the pairs
// (j, j + 8) of the tokens u and u + 4 of one 8-token group (u % 8 < 4) --
// both in the tile, since tiles are 8-aligned -- a token outside [off, off +
// nt) keeping its bits.  One thread per group: no two threads share a byte.
template <int TT>
__device__ void write_tile_1p25(uint8_t* kc, uint8_t* vc, int64_t tile_base, int off, int nt,
                                const uint16_t* kcodes, const uint16_t* vcodes) {
    static_assert(TT % 8 == 0, "whole 8-token groups per tile");
    constexpr int J = 16, W = 20;
    for (int idx = threadIdx.x; idx < nt * 4; idx += blockDim.x) {
        const int r = off + idx / 4, i = idx % 4;
        put_key_group_1p25(kc + (tile_base + r) * W, i, kcodes + r * J + 4 * i);
    }
    for (int idx = threadIdx.x; idx < (TT / 8) * 4 * 8; idx += blockDim.x) {
        const int ra = (idx / 32) * 8 + (idx / 8) % 4, rb = ra + 4, j = idx % 8;
        const bool ina = ra >= off && ra < off + nt, inb = rb >= off && rb < off + nt;
        if (!ina && !inb) continue;
        const int64_t bit = v_bit_1p25(tile_base + ra, j);          // a multiple of 40: five whole bytes
        if (ina) put_field(vc, bit, 20, (uint64_t)vcodes[ra * J + j] | ((uint64_t)vcodes[ra * J + j + 8] << 10));
        if (inb) put_field(vc, bit + 20, 20, (uint64_t)vcodes[rb * J + j] | ((uint64_t)vcodes[rb * J + j + 8] << 10));
    }
}

// Bulk quantization of a tile of TT positions of one (b, KV head) by the
// screen: block of 1024 threads; the key rows are rotated in LDS, then for
// keys and then values each wave screens sets of 4 points (token, sub-vector)
// against the whole codebook and refines.  Used for the 1.5-bit format
// (4096 entries), where it is 3x faster than the exact scan.
template <int FMT>
__global__ __launch_bounds__(1024) void quantize_screen_kernel(AppendArgs a) {
    using F = Fmt<FMT>;
    constexpr int E = F::E, DS = F::DS, J = F::J, W = F::W;
    constexpr int TT = AppendTile<FMT>::TT;
    constexpr int NWV = 16;
    __shared__ __align__(16) uint16_t book[E * DS];   // one codebook at a time (K, then V)
    __shared__ float cc[E];
    __shared__ float cb[2];
    __shared__ double x[TT * kHeadDim];
    __shared__ uint16_t codes[2][TT * J];

    const int h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tile_base = (a.start_pos / TT + blockIdx.x) * TT;
    const int lo = max(tile_base, a.start_pos);
    const int hi = min(tile_base + TT, a.start_pos + a.n_new);
    const int off = lo - tile_base;             // first valid row of the tile
    const int nt = hi - lo;                     // >= 1
    const int64_t stream = (int64_t)b * a.hkv + h;
    const int64_t row0 = stream * a.n_new + (lo - a.start_pos);   // input row of position lo

    // Keys: x = k / s, into LDS rows [off, off + nt), then the rotation.
    const float* s = a.smooth + (int64_t)h * kHeadDim;
    for (int idx = threadIdx.x; idx < nt * kHeadDim; idx += blockDim.x) {
        const int r = idx / kHeadDim, c = idx % kHeadDim;
        x[(off + r) * kHeadDim + c] = load_elem_d(a.k_new, (row0 + r) * kHeadDim + c, a.dtype) / (double)s[c];
    }
    __syncthreads();
    block_fwht(x + off * kHeadDim, nt);

    const int P = nt * J;                       // points per phase, contiguous from row off
    for (int phase = 0; phase < 2; ++phase) {
        if (phase == 1) {
            // Values; in the value-transform variant divided by s_v and rotated like the keys.
            const float* sv = a.v_smooth ? a.v_smooth + (int64_t)h * kHeadDim : nullptr;
            for (int idx = threadIdx.x; idx < nt * kHeadDim; idx += blockDim.x) {
                const int r = idx / kHeadDim, c = idx % kHeadDim;
                const double e = load_elem_d(a.v_new, (row0 + r) * kHeadDim + c, a.dtype);
                x[(off + r) * kHeadDim + c] = sv ? e / (double)sv[c] : e;
            }
            if (sv) {                                       // block-uniform
                __syncthreads();
                block_fwht(x + off * kHeadDim, nt);
            }
        }
        const uint4* src = (const uint4*)((phase == 0 ? a.k_book : a.v_book) + (int64_t)h * E * DS);
        for (int i = threadIdx.x; i < E * DS / 8; i += blockDim.x) ((uint4*)book)[i] = src[i];
        __syncthreads();
        book_norms<DS, E>(book, cc, cb);
        const double* xs = x + off * kHeadDim;
        constexpr int NP = 4;                     // points per screened set
        for (int base = wave * NP; base < P; base += NWV * NP) {
            const int np = min(NP, P - base);
            half4_t ahi[DS / 4], alo[DS / 4];
            bool oor;
            const double xn = screen_operands<DS, NP>(xs + base * DS, np, ahi, alo, oor);
            float m1[NP], m2[NP];
            int a1[NP];
#pragma unroll
            for (int q = 0; q < NP; ++q) { m1[q] = __builtin_inff(); m2[q] = __builtin_inff(); a1[q] = 0; }
            screen_set<DS, E, NP / 4>(ahi, alo, book, cc, 0, 1, m1, m2, a1);
            uint32_t fbmask = 0;
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                if (q < np) {
                    const float smin = wave_minf(m1[q]);
                    const double xq = __shfl(xn, q, 64);
                    const bool oq = __shfl((int)oor, q, 64) != 0;
                    const double thr = (double)smin + 3.0 * screen_tau(xq, cb);
                    const bool fb = oq || !(smin < __builtin_inff()) || __ballot((double)m2[q] <= thr) != 0;
                    if (fb) {
                        fbmask |= 1u << q;
                    } else {
                        const int code = refine_point<DS, E>(xs + (base + q) * DS, book, thr, false, m1[q], a1[q]);
                        if (lane == 0) codes[phase][off * J + base + q] = (uint16_t)code;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);      // one point at a time: bounded registers
            }
            while (fbmask) {                         // wave-uniform
                const int q = __builtin_ctz(fbmask);
                fbmask &= fbmask - 1;
                const int code = refine_point<DS, E>(xs + (base + q) * DS, book, 0.0, true, 0.0f, 0);
                if (lane == 0) codes[phase][off * J + base + q] = (uint16_t)code;
            }
        }
        __syncthreads();
    }

    // Write the codes of positions [lo, hi) in the cache layout.
    uint8_t* kc = a.k_codes + stream * (int64_t)a.cap * W;
    uint8_t* vc = a.v_codes + stream * (int64_t)a.cap * W;
    if (FMT == 0 || FMT == 4) {
        for (int idx = threadIdx.x; idx < nt * J; idx += blockDim.x) {
            const int r = off + idx / J, j = idx % J;
            const int64_t t = tile_base + r;
            kc[t * W + j] = (uint8_t)codes[0][r * J + j];
            vc[FMT == 0 ? v_code_offset_2bit(t, j) : v_code_offset_4bit(t, j)] = (uint8_t)codes[1][r * J + j];
        }
    } else if (FMT == 3) {
        write_tile_1p25<TT>(kc, vc, tile_base, off, nt, codes[0], codes[1]);
    } else {
        // Keys: sub-vectors (2i, 2i+1) of a token share 3 bytes.
        for (int idx = threadIdx.x; idx < nt * (J / 2); idx += blockDim.x) {
            const int r = off + idx / (J / 2), i = idx % (J / 2);
            const int64_t t = tile_base + r;
            const uint32_t c0 = codes[0][r * J + 2 * i], c1 = codes[0][r * J + 2 * i + 1];
            uint8_t* p = kc + t * W + 3 * i;
            p[0] = (uint8_t)(c0 & 0xff);
            p[1] = (uint8_t)((c0 >> 8) | ((c1 & 0xf) << 4));
            p[2] = (uint8_t)(c1 >> 4);
        }
        // Values: sub-vectors (j, j + J/2) of a token share 3 bytes.
        for (int idx = threadIdx.x; idx < nt * (J / 2); idx += blockDim.x) {
            const int r = off + idx / (J / 2), j = idx % (J / 2);
            const int64_t t = tile_base + r;
            const uint32_t c0 = codes[1][r * J + j], c1 = codes[1][r * J + j + J / 2];
            uint8_t* p = vc + v_pair_offset<FMT>(t, j);
            p[0] = (uint8_t)(c0 & 0xff);
            p[1] = (uint8_t)((c0 >> 8) | ((c1 & 0xf) << 4));
            p[2] = (uint8_t)(c1 >> 4);
        }
    }
}

// Bulk quantization by the exact scan (fp64 distances to every entry, over
// slices of the codebook): block of 256 threads per tile of TT positions.
// Used for the 256-entry books (2-bit, 4-bit), where the scan is cheaper than
// the screen's per-point reductions.
template <int FMT>
__global__ __launch_bounds__(256) void quantize_exact_kernel(AppendArgs a) {
    using F = Fmt<FMT>;
    constexpr int E = F::E, DS = F::DS, J = F::J, W = F::W;
    constexpr int TT = AppendTile<FMT>::TT;
    __shared__ double book[E * DS];             // one codebook at a time (K, then V), widened once
    __shared__ double xk[TT * kHeadDim];        // transformed keys of the tile
    __shared__ uint16_t codes[2][TT * J];
    __shared__ double red_d[256];
    __shared__ int red_i[256];

    const int h = blockIdx.y, b = blockIdx.z;
    const int tile_base = (a.start_pos / TT + blockIdx.x) * TT;
    const int lo = max(tile_base, a.start_pos);
    const int hi = min(tile_base + TT, a.start_pos + a.n_new);
    const int off = lo - tile_base;             // first valid row of the tile
    const int nt = hi - lo;                     // >= 1
    const int64_t stream = (int64_t)b * a.hkv + h;
    const int64_t row0 = stream * a.n_new + (lo - a.start_pos);   // input row of position lo

    // Keys: x = k / s, into LDS rows [off, off + nt).
    const float* s = a.smooth + (int64_t)h * kHeadDim;
    for (int idx = threadIdx.x; idx < nt * kHeadDim; idx += blockDim.x) {
        const int r = idx / kHeadDim, c = idx % kHeadDim;
        xk[(off + r) * kHeadDim + c] = load_elem_d(a.k_new, (row0 + r) * kHeadDim + c, a.dtype) / (double)s[c];
    }
    __syncthreads();
    block_fwht(xk + off * kHeadDim, nt);

    const int P = nt * J;                       // points per phase
    int ES = 1;                                 // centroid slices per point
    while (ES * 2 * P <= 256 && ES * 2 <= E / 16) ES *= 2;

    for (int phase = 0; phase < 2; ++phase) {
        if (phase == 1 && a.v_smooth != nullptr) {         // value-transform variant: x = H (v / s_v)
            const float* sv = a.v_smooth + (int64_t)h * kHeadDim;
            for (int idx = threadIdx.x; idx < nt * kHeadDim; idx += blockDim.x) {
                const int r = idx / kHeadDim, c = idx % kHeadDim;
                xk[(off + r) * kHeadDim + c] = load_elem_d(a.v_new, (row0 + r) * kHeadDim + c, a.dtype) / (double)sv[c];
            }
            __syncthreads();
            block_fwht(xk + off * kHeadDim, nt);
        }
        const uint16_t* src = (phase == 0 ? a.k_book : a.v_book) + (int64_t)h * E * DS;
        for (int i = threadIdx.x; i < E * DS; i += blockDim.x) book[i] = (double)half_bits_to_float(src[i]);
        __syncthreads();
        const int items = P * ES;
        for (int it = threadIdx.x; it < items; it += blockDim.x) {
            const int pt = it / ES, sl = it % ES;
            const int r = pt / J, j = pt % J;
            double x[DS];
            if (phase == 0 || a.v_smooth != nullptr) {
#pragma unroll
                for (int i = 0; i < DS; ++i) x[i] = xk[(off + r) * kHeadDim + j * DS + i];
            } else {
#pragma unroll
                for (int i = 0; i < DS; ++i) x[i] = load_elem_d(a.v_new, (row0 + r) * kHeadDim + j * DS + i, a.dtype);
            }
            double best;
            int idx;
            argmin_range<DS>(x, book, sl * (E / ES), (sl + 1) * (E / ES), best, idx);
            if (ES == 1) {
                codes[phase][(off + r) * J + j] = (uint16_t)idx;
            } else {
                red_d[it] = best;
                red_i[it] = idx;
            }
        }
        __syncthreads();
        if (ES > 1) {
            for (int pt = threadIdx.x; pt < P; pt += blockDim.x) {
                double best = red_d[pt * ES];
                int idx = red_i[pt * ES];
                for (int sl = 1; sl < ES; ++sl)
                    if (red_d[pt * ES + sl] < best) { best = red_d[pt * ES + sl]; idx = red_i[pt * ES + sl]; }
                codes[phase][(off + pt / J) * J + pt % J] = (uint16_t)idx;
            }
        }
        __syncthreads();
    }

    // Write the codes of positions [lo, hi) in the cache layout.
    uint8_t* kc = a.k_codes + stream * (int64_t)a.cap * W;
    uint8_t* vc = a.v_codes + stream * (int64_t)a.cap * W;
    if (FMT == 0 || FMT == 4) {
        for (int idx = threadIdx.x; idx < nt * J; idx += blockDim.x) {
            const int r = off + idx / J, j = idx % J;
            const int64_t t = tile_base + r;
            kc[t * W + j] = (uint8_t)codes[0][r * J + j];
            vc[FMT == 0 ? v_code_offset_2bit(t, j) : v_code_offset_4bit(t, j)] = (uint8_t)codes[1][r * J + j];
        }
    } else if (FMT == 3) {
        write_tile_1p25<TT>(kc, vc, tile_base, off, nt, codes[0], codes[1]);
    } else {
        // Keys: sub-vectors (2i, 2i+1) of a token share 3 bytes.
        for (int idx = threadIdx.x; idx < nt * (J / 2); idx += blockDim.x) {
            const int r = off + idx / (J / 2), i = idx % (J / 2);
            const int64_t t = tile_base + r;
            const uint32_t c0 = codes[0][r * J + 2 * i], c1 = codes[0][r * J + 2 * i + 1];
            uint8_t* p = kc + t * W + 3 * i;
            p[0] = (uint8_t)(c0 & 0xff);
            p[1] = (uint8_t)((c0 >> 8) | ((c1 & 0xf) << 4));
            p[2] = (uint8_t)(c1 >> 4);
        }
        // Values: sub-vectors (j, j + J/2) of a token share 3 bytes.
        for (int idx = threadIdx.x; idx < nt * (J / 2); idx += blockDim.x) {
            const int r = off + idx / (J / 2), j = idx % (J / 2);
            const int64_t t = tile_base + r;
            const uint32_t c0 = codes[1][r * J + j], c1 = codes[1][r * J + j + J / 2];
            uint8_t* p = vc + v_pair_offset<FMT>(t, j);
            p[0] = (uint8_t)(c0 & 0xff);
            p[1] = (uint8_t)((c0 >> 8) | ((c1 & 0xf) << 4));
            p[2] = (uint8_t)(c1 >> 4);
        }
    }
}

// ------------------------------------------------- append of a single token

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// |c|^2 and x.c for one codebook entry of DS fp16 values (LDS, 8- or
// 16-byte aligned) on the dot units: fp16 pairs, fp32 sums.
template <int DS>
__device__ __forceinline__ void screen_dot(const uint16_t* c, const half2_t (&xh)[DS / 2], float& n2, float& xc) {
    uint32_t w[DS / 2];
    if constexpr (DS == 8) {
        const uint4 v = *(const uint4*)c;
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
        static_assert(DS == 4, "screen_dot: 4 or 8 values");
        const uint2 v = *(const uint2*)c;
        w[0] = v.x; w[1] = v.y;
    }
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int i = 0; i < DS / 2; ++i) {
        const half2_t ch = __builtin_bit_cast(half2_t, w[i]);
        a = __builtin_amdgcn_fdot2(ch, ch, a, false);
        b = __builtin_amdgcn_fdot2(xh[i], ch, b, false);
    }
    n2 = a;
    xc = b;
}

// Blocks per key (and per value) of the one-token append: a 4096-entry search
// is split over 4 blocks of 4 sub-vectors each, so the grid fills the GPU.
template <int FMT> struct TokenSplit {                  // 256 entries: 1 block, 1024: 2, 4096: 4
    static constexpr int P = (FMT == 0 || FMT == 4) ? 1 : (FMT == 3 ? 2 : 4);
};

// The per-step append (one new token per sequence), latency-bound: grid
// (2P, Hkv, B), block x / P = 0 codes the key, 1 the value, x % P = part p
// codes J / P of the sub-vectors (keys: consecutive ones; 1.5-bit values: the
// pairs (i, i + 8) that share three bytes, kept in one block).  The codebook
// and the row are staged in LDS at once; the key blocks rotate the key with
// one wave (the same butterflies as block_fwht, stage h exchanged between
// lanes l and l ^ h, so the result is identical).  Each sub-vector's search
// runs over ES interleaved slices of the codebook, one per thread; the slices'
// minima are merged as (distance, index) pairs, lowest pair first, which is
// the scan's lowest-index minimum whatever the merge order.
template <int FMT>
// Two 1024-thread blocks per CU need at most 64 VGPRs (the 3-bit search keeps
// 32 screened distances per thread; the cap costs it a few spilled dwords).
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8))) void quantize_token_kernel(AppendArgs a) {
    using F = Fmt<FMT>;
    constexpr int E = F::E, DS = F::DS, J = F::J, W = F::W;
    constexpr int NT = 1024, P = TokenSplit<FMT>::P;
    constexpr int JB = J / P;                   // sub-vectors per block
    constexpr int ES = NT / JB;                 // slices per sub-vector
    constexpr int EPS = E / ES;                 // centroids per slice
    constexpr int L = ES < 64 ? ES : 64;        // lanes of one sub-vector in a wave
    constexpr int WPS = ES / L;                 // waves per sub-vector
    static_assert(JB % 2 == 0 && E % ES == 0 && (L & (L - 1)) == 0, "token search shape");
    __shared__ __align__(16) uint16_t book[E * DS];
    __shared__ double x[kHeadDim];
    __shared__ double part_d[NT / 64];
    __shared__ int part_i[NT / 64];
    __shared__ float part_m[NT / 64], part_c[NT / 64];
    __shared__ uint16_t codes[JB];

    const int ph = blockIdx.x / P, part = blockIdx.x % P, h = blockIdx.y, b = blockIdx.z;
    const int64_t stream = (int64_t)b * a.hkv + h;
    if (a.q_prime != nullptr && ph == 0 && part == 0) {   // decode-step prologue, before the key's own work:
        const int G = a.hq / a.hkv, w = (int)(threadIdx.x >> 6) - 1;
        if (w >= 0 && w < G) {                  // waves 1..G: q' of this head's query group
            const int64_t vec = (int64_t)b * a.hq + h * G + w;
            transform_query_wave((const char*)a.q + vec * kHeadDim * (a.dtype == 0 ? 2 : 4), a.dtype,
                                 a.smooth + (int64_t)h * kHeadDim, a.q_prime + vec * kHeadDim, threadIdx.x & 63);
        }
        if (threadIdx.x == 0) a.arrivals[stream] = 0;
        if (threadIdx.x == 0 && h == 0 && a.seq_lens_out != nullptr) {
            const int64_t pos = a.positions[b];
            a.seq_lens_out[b] = (int32_t)(pos < 0 ? 0 : (pos >= a.cap ? a.cap : pos + 1));
        }
    }
    // Position of the token: uniform, or per sequence (a position outside the
    // cache is skipped, block-uniformly, so nothing is written out of bounds).
    const int64_t t = a.positions ? (int64_t)a.positions[b] : (int64_t)a.start_pos;
    if (t < 0 || t >= a.cap) return;
    // Sub-vector j of the block's jj-th.
    // 12-bit values: the block's JB / 2 low sub-vectors and their partners J / 2 further.
    auto sub_of = [&](int jj) -> int {
        if (FMT != 0 && FMT != 4 && ph == 1) return (JB / 2) * part + jj % (JB / 2) + (J / 2) * (jj / (JB / 2));
        return part * JB + jj;
    };
    {
        const uint4* src = (const uint4*)((ph == 0 ? a.k_book : a.v_book) + (int64_t)h * E * DS);
        for (int i = threadIdx.x; i < E * DS / 8; i += NT) ((uint4*)book)[i] = src[i];
        if (threadIdx.x < kHeadDim) {
            const int c = threadIdx.x;
            // Keys, and values of the value-transform variant: divided by their scales.
            const float* div = ph == 0 ? a.smooth : a.v_smooth;
            const double e = load_elem_d(ph == 0 ? a.k_new : a.v_new, stream * kHeadDim + c, a.dtype);
            x[c] = div ? e / (double)div[(int64_t)h * kHeadDim + c] : e;
        }
    }
    __syncthreads();
    if ((ph == 0 || a.v_smooth != nullptr) && threadIdx.x < 64)   // the rotation (block-uniform)
        rotate_row_wave(x, threadIdx.x);
    __syncthreads();
    {
        const int jj = threadIdx.x / ES, sl = threadIdx.x % ES;
        const int j = sub_of(jj);
        double xs[DS];
#pragma unroll
        for (int i = 0; i < DS; ++i) xs[i] = x[j * DS + i];
        // Slice sl = entries sl, sl + ES, sl + 2 ES, ...: at every step the
        // lanes read consecutive entries (no LDS bank conflicts).
        double best = __builtin_inf();
        int idx = sl;
        bool exact = FMT == 0 || FMT == 4;
        if constexpr (FMT != 0 && FMT != 4) {
            // 4096 entries: a screen on the dot units, then the pinned fp64
            // distance for the candidates only.  Up to the common |x|^2, the
            // distance is s = |c|^2 - 2 x.c; the screen takes x rounded to
            // fp16 and fp32 sums of fp16 products (exact products; at most two
            // roundings per pair).  With R = |x| + max_e |c_e| the screened s32
            // is within 2^-11.9 R^2 + 2^-11.5 R + 2^-25 of s: 2^-10.9 |x_i| for
            // x's rounding, 2^-14 per coordinate if the unit flushed fp16
            // subnormals (of x or c), (DS + 3) 2^-24 R^2 for the sums.  tau =
            // 2^-11 (R^2 + R) + 2^-24 covers that and the fp64 rounding of the
            // pinned distance, so the pinned minimum and every entry tied with
            // it have s32 <= m + 2 tau (m = the smallest s32): refining those
            // entries and taking the lowest (distance, index) gives the scan's
            // code.  A coordinate that is not finite or reaches 2^15 (fp16
            // overflow), or no finite s32, sends the sub-vector to the exact scan.
            half2_t xh[DS / 2];
            float s32[EPS];
            double xn2 = 0.0;
            bool ok = true;
#pragma unroll
            for (int i = 0; i < DS; ++i) {
                xn2 = xn2 + xs[i] * xs[i];
                ok = ok && __builtin_fabs(xs[i]) < 0x1p15;
            }
#pragma unroll
            for (int i = 0; i < DS / 2; ++i)
                xh[i] = half2_t{(_Float16)(float)xs[2 * i], (_Float16)(float)xs[2 * i + 1]};
            float m = __builtin_inff(), c2 = 0.0f;
#pragma unroll
            for (int k = 0; k < EPS; ++k) {
                float n2, xc;
                screen_dot<DS>(book + (sl + k * ES) * DS, xh, n2, xc);
                s32[k] = __builtin_fmaf(-2.0f, xc, n2);
                m = fminf(m, s32[k]);
                c2 = fmaxf(c2, n2);
            }
            // The smallest s32 and the largest |c|^2 over the sub-vector's ES slices.
#pragma unroll
            for (int o = 1; o < L; o <<= 1) {
                m = fminf(m, __shfl_xor(m, o, 64));
                c2 = fmaxf(c2, __shfl_xor(c2, o, 64));
            }
            if constexpr (WPS > 1) {
                if ((threadIdx.x & 63) == 0) {
                    part_m[threadIdx.x >> 6] = m;
                    part_c[threadIdx.x >> 6] = c2;
                }
                __syncthreads();
#pragma unroll
                for (int w = 0; w < WPS; ++w) {
                    m = fminf(m, part_m[jj * WPS + w]);
                    c2 = fmaxf(c2, part_c[jj * WPS + w]);
                }
            }
            exact = !ok || !(__builtin_fabsf(m) < __builtin_inff());   // uniform over the sub-vector
            if (!exact) {
                // |c| <= sqrt(n2) up to the sums' rounding and flushed subnormals.
                const double r = __builtin_sqrt(xn2) + __builtin_sqrt((double)c2 * (1.0 + 0x1p-16)) + 0x1p-12;
                const double thr = (double)m + 2.0 * (0x1p-11 * (r * r + r) + 0x1p-24);
#pragma unroll
                for (int k = 0; k < EPS; ++k) {
                    if ((double)s32[k] <= thr) {
                        const int e = sl + k * ES;
                        const double d = dist_h<DS>(xs, book + e * DS);
                        if (d < best) { best = d; idx = e; }
                    }
                }
            }
        }
        if (exact) {
            for (int k = 0; k < EPS; ++k) {
                const int e = sl + k * ES;
                const double d = dist_h<DS>(xs, book + e * DS);
                if (d < best) { best = d; idx = e; }
            }
        }
        group_argmin<L>(best, idx);
        if (WPS == 1) {
            if (sl == 0) codes[jj] = (uint16_t)idx;
        } else if ((threadIdx.x & 63) == 0) {
            part_d[threadIdx.x >> 6] = best;
            part_i[threadIdx.x >> 6] = idx;
        }
    }
    __syncthreads();
    if (WPS > 1 && threadIdx.x < JB) {
        const int jj = threadIdx.x;
        double best = part_d[jj * WPS];
        int idx = part_i[jj * WPS];
        for (int w = 1; w < WPS; ++w) {
            const double d = part_d[jj * WPS + w];
            const int i = part_i[jj * WPS + w];
            if (d < best || (d == best && i < idx)) { best = d; idx = i; }
        }
        codes[jj] = (uint16_t)idx;
    }
    if (WPS > 1) __syncthreads();
    // The token's 64-token block: in the stream, or (paged) the pool block the
    // table names, clamped to the pool; u = position inside the block.
    uint8_t* kblk;
    uint8_t* vblk;
    if (a.block_table) {
        int blk = a.block_table[stream * (int64_t)(a.cap >> 6) + (t >> 6)];
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        kblk = a.k_codes + (int64_t)blk * (64 * W);
        vblk = a.v_codes + (int64_t)blk * (64 * W);
    } else {
        kblk = a.k_codes + stream * (int64_t)a.cap * W + (t >> 6) * (64 * W);
        vblk = a.v_codes + stream * (int64_t)a.cap * W + (t >> 6) * (64 * W);
    }
    const int u = (int)(t & 63);
    if (FMT == 0 || FMT == 4) {
        if (threadIdx.x < JB) {
            const int j = sub_of(threadIdx.x);
            if (ph == 0) kblk[u * W + j] = (uint8_t)codes[threadIdx.x];
            else vblk[FMT == 0 ? v_code_offset_2bit(u, j) : v_code_offset_4bit(u, j)] = (uint8_t)codes[threadIdx.x];
        }
    } else if (FMT == 3) {
        // Keys: the block's JB consecutive sub-vectors, whole 5-byte groups of
        // the token.  Values: the pairs (j, j + 8), 20 bits each, sharing a
        // byte with token u +- 4, whose bits are kept (one token per stream
        // per call: no other writer of that byte).
        if (ph == 0 && threadIdx.x < JB / 4)
            put_key_group_1p25(kblk + u * W, (part * JB) / 4 + (int)threadIdx.x, codes + 4 * threadIdx.x);
        if (ph == 1 && threadIdx.x < JB / 2) {
            const int m = threadIdx.x;
            put_field(vblk, v_bit_1p25(u, sub_of(m)), 20, (uint64_t)codes[m] | ((uint64_t)codes[m + JB / 2] << 10));
        }
    } else if (threadIdx.x < JB / 2) {
        // Keys: sub-vectors (2i, 2i+1) share 3 bytes (the block's jj = 2m, 2m+1);
        // values: (i, i + J/2) (the block's jj = m, m + JB/2).
        const int m = threadIdx.x;
        const int jj0 = ph == 0 ? 2 * m : m, jj1 = ph == 0 ? 2 * m + 1 : m + JB / 2;
        const uint32_t c0 = codes[jj0], c1 = codes[jj1];
        const int j0 = sub_of(jj0);
        uint8_t* p = ph == 0 ? kblk + u * W + 3 * (j0 >> 1) : vblk + v_pair_offset<FMT>(u, j0);
        p[0] = (uint8_t)(c0 & 0xff);
        p[1] = (uint8_t)((c0 >> 8) | ((c1 & 0xf) << 4));
        p[2] = (uint8_t)(c1 >> 4);
    }
}


// --------------------------------------------------------- smoothing scales

// s[h][c] = fp32 nearest sqrt(max_t |k[h][t][c]|).  The fp64 root is checked
// against the two fp32 rounding midpoints with exact fp64 squares, so the
// result is the correctly rounded fp32 root whatever the accuracy of sqrt.
__global__ __launch_bounds__(128) void smooth_scales_kernel(int n_cal, const void* k_cal, int dtype, float* smooth) {
    const int h = blockIdx.x, c = threadIdx.x;
    float m = 0.0f;
    const int64_t base = (int64_t)h * n_cal * kHeadDim + c;
    for (int t = 0; t < n_cal; ++t) m = fmaxf(m, fabsf(load_elem(k_cal, base + (int64_t)t * kHeadDim, dtype)));
    const double md = (double)m;
    float r = (float)sqrt(md);
    // Correct to the nearest fp32: midpoints have 25 significant bits, their squares are exact in fp64.
    for (int it = 0; it < 2; ++it) {
        const float up = nextafterf(r, __builtin_inff());
        const double mid_up = 0.5 * ((double)r + (double)up);
        if (md >= mid_up * mid_up) { r = up; continue; }
        const float dn = nextafterf(r, 0.0f);
        const double mid_dn = 0.5 * ((double)r + (double)dn);
        if (r > 0.0f && md < mid_dn * mid_dn) { r = dn; continue; }
        break;
    }
    smooth[h * kHeadDim + c] = r;
}

// ------------------------------------------------------------ codebook training

// Points for K-Means: rotated keys or raw values, fp64 [n_cal][128].
__global__ __launch_bounds__(256) void calib_points_kernel(TrainArgs a) {
    constexpr int R = 8;                               // rows per block
    __shared__ double x[R * kHeadDim];
    const int r0 = blockIdx.x * R;
    const int nr = min(R, a.n_cal - r0);
    for (int idx = threadIdx.x; idx < nr * kHeadDim; idx += blockDim.x) {
        const int r = idx / kHeadDim, c = idx % kHeadDim;
        const double v = load_elem_d(a.rows, (int64_t)(r0 + r) * kHeadDim + c, a.dtype);
        x[idx] = a.is_key ? v / (double)a.smooth[c] : v;
    }
    __syncthreads();
    if (a.is_key) block_fwht(x, nr);
    for (int idx = threadIdx.x; idx < nr * kHeadDim; idx += blockDim.x)
        a.points[(int64_t)r0 * kHeadDim + idx] = x[idx];
}

template <int DS>
__global__ __launch_bounds__(256) void kmeans_init_kernel(const double* pts, int64_t n, const int64_t* init, int E,
                                                          double* cent) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= E * DS) return;
    int64_t p = init[i / DS];
    p = p < 0 ? 0 : (p >= n ? n - 1 : p);
    cent[i] = pts[p * DS + i % DS];
}

// Assignment: one point per thread, centroids staged through LDS in chunks;
// chunks are visited in increasing index order with strict "<".
template <int DS>
__global__ __launch_bounds__(256) void kmeans_assign_kernel(const double* pts, int64_t n, const double* cent,
                                                            int E, int32_t* assign) {
    constexpr int CH = 8192 / DS;                      // centroids per chunk (64 KB)
    __shared__ double c[CH * DS];
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    double x[DS];
    if (p < n) {
#pragma unroll
        for (int i = 0; i < DS; ++i) x[i] = pts[p * DS + i];
    }
    double best = __builtin_inf();
    int idx = 0;
    for (int e0 = 0; e0 < E; e0 += CH) {
        const int ne = min(CH, E - e0);
        __syncthreads();
        for (int i = threadIdx.x; i < ne * DS; i += blockDim.x) c[i] = cent[(int64_t)e0 * DS + i];
        __syncthreads();
        if (p < n) {
            for (int e = 0; e < ne; ++e) {
                const double d = dist_f64<DS>(x, c + e * DS);
                if (d < best) { best = d; idx = e0 + e; }
            }
        }
    }
    if (p < n) assign[p] = idx;
}

// Update: one wave per centroid scans the assignment in point order; lane i < DS
// keeps the running fp64 sum of dimension i, so every sum is taken in
// increasing point order.
template <int DS>
__global__ __launch_bounds__(256) void kmeans_update_kernel(const double* pts, int64_t n, const int32_t* assign,
                                                            int E, double* cent) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    double sum = 0.0;
    int64_t count = 0;
    for (int64_t base = 0; base < n; base += 64) {
        const int64_t p = base + lane;
        const bool hit = p < n && assign[p] == e;
        uint64_t mask = __ballot(hit);
        count += __popcll(mask);
        while (mask) {
            const int l = __ffsll((unsigned long long)mask) - 1;
            mask &= mask - 1;
            if (lane < DS) sum = sum + pts[(base + l) * DS + lane];
        }
    }
    if (count > 0 && lane < DS) cent[(int64_t)e * DS + lane] = sum / (double)count;
}

// fp64 -> fp16, round to nearest, ties to even; overflow to infinity.
__device__ uint16_t double_to_half_rne(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000);
    const uint64_t mag = u & 0x7fffffffffffffffull;
    if (mag > 0x7ff0000000000000ull) return (uint16_t)(sign | 0x7e00);        // NaN
    const double a = __builtin_bit_cast(double, mag);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (a < 0x1p-14) {                                                        // subnormal halves
        const double q = a * 0x1p24;                                          // exact scaling
        double n = __builtin_rint(q);                                         // rint: ties to even
        return (uint16_t)(sign | (uint16_t)n);
    }
    const int e = (int)((mag >> 52) & 0x7ff) - 1023;                          // a in [2^e, 2^(e+1))
    const double q = a * __builtin_ldexp(1.0, 10 - e);                        // in [1024, 2048)
    const double n = __builtin_rint(q);                                       // may reach 2048
    const uint32_t m = (uint32_t)n;
    if (m == 2048) return (uint16_t)(sign | ((e + 16) << 10));
    return (uint16_t)(sign | ((e + 15) << 10) | (m - 1024));
}

__global__ __launch_bounds__(256) void round_book_kernel(const double* cent, int count, uint16_t* book) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) book[i] = double_to_half_rne(cent[i]);
}

template <int FMT>
hipError_t train_codebook(const TrainArgs& a, hipStream_t stream) {
    using F = Fmt<FMT>;
    constexpr int E = F::E, DS = F::DS, J = F::J;
    const int64_t n = (int64_t)a.n_cal * J;
    hipLaunchKernelGGL(calib_points_kernel, dim3((a.n_cal + 7) / 8), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(kmeans_init_kernel<DS>, dim3((E * DS + 255) / 256), dim3(256), 0, stream,
                       (const double*)a.points, n, a.init, E, a.centroids);
    const int ablocks = (int)((n + 255) / 256);
    for (int it = 0; it < a.iters; ++it) {
        hipLaunchKernelGGL(kmeans_assign_kernel<DS>, dim3(ablocks), dim3(256), 0, stream,
                           (const double*)a.points, n, (const double*)a.centroids, E, a.assign);
        hipLaunchKernelGGL(kmeans_update_kernel<DS>, dim3(E / 4), dim3(256), 0, stream,
                           (const double*)a.points, n, (const int32_t*)a.assign, E, a.centroids);
    }
    hipLaunchKernelGGL(round_book_kernel, dim3((E * DS + 255) / 256), dim3(256), 0, stream,
                       (const double*)a.centroids, E * DS, a.book);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_append(const AppendArgs& a, hipStream_t stream) {
    static_assert(AppendTile<0>::TT == AppendTile<4>::TT && AppendTile<1>::TT == AppendTile<2>::TT &&
                  AppendTile<1>::TT == AppendTile<3>::TT, "tile sizes by book size");
    const int TT = (a.fmt == 0 || a.fmt == 4) ? AppendTile<0>::TT : AppendTile<1>::TT;
    const int first = a.start_pos / TT, last = (a.start_pos + a.n_new - 1) / TT;
    const dim3 grid(last - first + 1, a.hkv, a.batch);
    if (a.n_new == 1 || a.positions) {
        const int P = a.fmt == 0 ? TokenSplit<0>::P
                    : (a.fmt == 1 ? TokenSplit<1>::P
                                  : (a.fmt == 2 ? TokenSplit<2>::P : (a.fmt == 3 ? TokenSplit<3>::P : TokenSplit<4>::P)));
        const dim3 g1(2 * P, a.hkv, a.batch);
        if (a.fmt == 0) hipLaunchKernelGGL(quantize_token_kernel<0>, g1, dim3(1024), 0, stream, a);
        else if (a.fmt == 1) hipLaunchKernelGGL(quantize_token_kernel<1>, g1, dim3(1024), 0, stream, a);
        else if (a.fmt == 2) hipLaunchKernelGGL(quantize_token_kernel<2>, g1, dim3(1024), 0, stream, a);
        else if (a.fmt == 3) hipLaunchKernelGGL(quantize_token_kernel<3>, g1, dim3(1024), 0, stream, a);
        else hipLaunchKernelGGL(quantize_token_kernel<4>, g1, dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    if (a.fmt == 0) hipLaunchKernelGGL(quantize_exact_kernel<0>, grid, dim3(256), 0, stream, a);
    else if (a.fmt == 1) hipLaunchKernelGGL(quantize_screen_kernel<1>, grid, dim3(1024), 0, stream, a);
    else if (a.fmt == 2) hipLaunchKernelGGL(quantize_screen_kernel<2>, grid, dim3(1024), 0, stream, a);
    else if (a.fmt == 3) hipLaunchKernelGGL(quantize_screen_kernel<3>, grid, dim3(1024), 0, stream, a);
    else hipLaunchKernelGGL(quantize_exact_kernel<4>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_smooth_scales(int hkv, int n_cal, const void* k_cal, int dtype, float* smooth, hipStream_t stream) {
    hipLaunchKernelGGL(smooth_scales_kernel, dim3(hkv), dim3(128), 0, stream, n_cal, k_cal, dtype, smooth);
    return hipGetLastError();
}

hipError_t launch_train_codebook(const TrainArgs& a, hipStream_t stream) {
    if (a.fmt == 0) return train_codebook<0>(a, stream);
    if (a.fmt == 3) return train_codebook<3>(a, stream);
    if (a.fmt == 4) return train_codebook<4>(a, stream);
    return a.fmt == 1 ? train_codebook<1>(a, stream) : train_codebook<2>(a, stream);
}

}  // namespace vqkv
