// decode.hip -- split-context decode attention that reads the VQ codes directly,
// and the log-sum-exp combine of the splits.
//
// VecInfer abstract (arXiv 2510.06175): a kernel that fuses dequantization
// into the attention computation so that only the compact codes are read
// from memory.  Decode attention is bound by memory traffic (every step
// re-reads the whole cache), so the design moves the codes once, with wide
// coalesced loads, and does all dequantization from LDS.
//
// Work split.  Grid (splits, Hkv, B): one work-group per (batch, KV head,
// token range).  The G = Hq / Hkv query heads of a KV head share the pass
// over its codes.  Each wave takes 64-token tiles of the range in turn and
// keeps its own online-softmax state (running max m, lane-partial sums l,
// output accumulators); the waves are merged at the end and the split writes
// (o normalized, lse) to the workspace.  Scores carry the factor
// sm_scale * log2(e), so exp2 is the exponential and lse is in log2 units.
//
// Per tile, lane = token for the scores (each lane sums its token's J
// sub-vector contributions), then lane = (sub-vector j, token group) for the
// value accumulation (each lane owns dims [j*dsub, (j+1)*dsub) of all G
// outputs).  The probabilities move between the two mappings through a
// per-wave LDS buffer.  Value codes are stored blocked by sub-vector so that
// this second mapping also reads contiguous 16-byte chunks.
//
// Scores, two ways (chosen by measurement):
//   * score table (2-bit, G <= 4): per work-group, L[j][e][g] =
//     c * q'_g[4j..4j+3] . C_K[e] for all 32 x 256 (j, e); a token's score is
//     then 32 table reads and adds (one 16-byte read serves all heads);
//   * gather: the token's centroids are read from the LDS codebook and dotted
//     with q' (held in LDS, pre-scaled) -- needed for 1.5-bit, where the table
//     would be 16 x 4096 x G floats.
#include "device_util.h"
#include "internal.h"

namespace vqkv {

namespace {

constexpr float kNegInf = -__builtin_inff();

// Bytes of the per-(b, h) code stream per token.
template <int FMT> struct DFmt;
template <> struct DFmt<0> { static constexpr int E = 256, DS = 4, J = 32, W = 32; };
template <> struct DFmt<1> { static constexpr int E = 4096, DS = 8, J = 16, W = 24; };

// Byte k (compile-time after unrolling) of a little-endian dword array.
template <int N>
__device__ __forceinline__ uint32_t byte_at(const uint32_t (&w)[N], int k) {
    return (w[k >> 2] >> (8 * (k & 3))) & 0xffu;
}

// 12-bit code `i` of a packed pair array (pairs (2m, 2m+1) in bytes 3m..3m+2).
template <int N>
__device__ __forceinline__ uint32_t code12_at(const uint32_t (&w)[N], int i) {
    const int m = i >> 1;
    const uint32_t b0 = byte_at(w, 3 * m), b1 = byte_at(w, 3 * m + 1), b2 = byte_at(w, 3 * m + 2);
    return (i & 1) ? ((b1 >> 4) | (b2 << 4)) : (b0 | ((b1 & 0xfu) << 8));
}

// Online-softmax update for one tile: sc holds this lane's G scores (log2 units,
// -inf for masked tokens); returns p and rescales l and acc.
template <int G, int NACC>
__device__ __forceinline__ void softmax_tile(float (&sc)[G], float (&m)[G], float (&l)[G],
                                             float (&acc)[G][NACC], float (&p)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float tm = wave_max(sc[g]);
        const float mn = fmaxf(m[g], tm);
        if (mn != m[g]) {                                   // wave-uniform
            const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
            l[g] *= alpha;
#pragma unroll
            for (int i = 0; i < NACC; ++i) acc[g][i] *= alpha;
            m[g] = mn;
        }
        p[g] = __builtin_amdgcn_exp2f(sc[g] - m[g]);
        l[g] += p[g];
    }
}

// Merge the NW waves' states and write the split's (o, lse).  Every thread of
// the block calls this.  `scratch` must hold NW * G * (128 + 2) floats and be
// free for reuse (caller synchronizes before).  Lanes [0, 128 / DS) of each
// wave hold the wave's (already token-group-reduced) accumulators for dims
// [lane * DS, lane * DS + DS).
template <int G, int DS, int NW>
__device__ __forceinline__ void merge_and_store(float* scratch, const float (&m)[G], const float (&l)[G],
                                                const float (&acc)[G][DS], const DecodeArgs& a,
                                                int b, int h, int s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float* mo = scratch;                                   // [NW][G][128]
    float* ml = scratch + NW * G * kHeadDim;               // [NW][G][2]
    if (lane < kHeadDim / DS) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < DS; ++i) mo[(wave * G + g) * kHeadDim + lane * DS + i] = acc[g][i];
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ml[(wave * G + g) * 2] = m[g];
            ml[(wave * G + g) * 2 + 1] = l[g];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += NW * 64) {
        const int g = idx / kHeadDim, d = idx % kHeadDim;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ml[(w * G + g) * 2]);
        float o = 0.0f, lse = kNegInf;
        if (M != kNegInf) {
            float L = 0.0f, O = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = ml[(w * G + g) * 2];
                const float f = mw == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
                L += f * ml[(w * G + g) * 2 + 1];
                O += f * mo[(w * G + g) * kHeadDim + d];
            }
            o = O / L;
            lse = M + __builtin_log2f(L);
        }
        const int64_t row = ((int64_t)b * a.hq + h * G + g) * a.splits + s;
        a.part_o[row * kHeadDim + d] = o;
        if (d == 0) a.part_lse[row] = lse;
    }
}

// ------------------------------------------------------------ score-table path

template <int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_table_kernel(DecodeArgs a) {
    constexpr int GP = G == 3 ? 4 : G;                     // table entry width (floats)
    constexpr int J = 32, E = 256;
    __shared__ __align__(16) float table[J * E * GP];
    __shared__ __align__(16) uint2 vbook[E];               // 4 fp16 per entry
    __shared__ __align__(16) float pbuf[NW][64 * GP];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t_begin = s * a.chunk;
    const int t_end = min(a.seq_len, t_begin + a.chunk);

    const uint2* vb = (const uint2*)(a.v_book + (int64_t)h * E * 4);
    for (int i = threadIdx.x; i < E; i += NW * 64) vbook[i] = vb[i];
    {
        const uint2* kb = (const uint2*)(a.k_book + (int64_t)h * E * 4);
        const float* qp = a.q_prime + ((int64_t)b * a.hq + h * G) * kHeadDim;
        for (int idx = threadIdx.x; idx < J * E; idx += NW * 64) {
            const int j = idx >> 8, e = idx & 255;
            const uint2 c = kb[e];
            const float c0 = lo_half(c.x), c1 = hi_half(c.x), c2 = lo_half(c.y), c3 = hi_half(c.y);
            float v[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                if (g < G) {
                    const float4 q = *(const float4*)(qp + g * kHeadDim + 4 * j);
                    v[g] = (q.x * c0 + q.y * c1 + q.z * c2 + q.w * c3) * a.qscale;
                } else {
                    v[g] = 0.0f;
                }
            }
            if constexpr (GP == 4) *(float4*)(table + idx * 4) = make_float4(v[0], v[1], v[2], v[3]);
            else if constexpr (GP == 2) *(float2*)(table + idx * 2) = make_float2(v[0], v[1]);
            else table[idx] = v[0];
        }
    }
    __syncthreads();

    float m[G], l[G], acc[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;
    }
    const int64_t stream = (int64_t)b * a.hkv + h;
    const uint8_t* kbase = a.k_codes + stream * (int64_t)a.cap * 32;
    const uint8_t* vbase = a.v_codes + stream * (int64_t)a.cap * 32;
    const int jv = lane & 31, half = lane >> 5;
    float* pw = pbuf[wave];

    for (int tile = t_begin + wave * 64; tile < t_end; tile += NW * 64) {
        const int t = tile + lane;
        uint32_t kw[8], vw[8];
        {
            const uint4* kc = (const uint4*)(kbase + (int64_t)t * 32);
            const uint4 k0 = kc[0], k1 = kc[1];
            kw[0] = k0.x; kw[1] = k0.y; kw[2] = k0.z; kw[3] = k0.w;
            kw[4] = k1.x; kw[5] = k1.y; kw[6] = k1.z; kw[7] = k1.w;
            const uint4* vc = (const uint4*)(vbase + (int64_t)(tile + half * 32) * 32 + jv * 32);
            const uint4 v0 = vc[0], v1 = vc[1];
            vw[0] = v0.x; vw[1] = v0.y; vw[2] = v0.z; vw[3] = v0.w;
            vw[4] = v1.x; vw[5] = v1.y; vw[6] = v1.z; vw[7] = v1.w;
        }
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = 0.0f;
        // One dword (four sub-vectors) per step; the code words rotate through
        // kw[0] so that indexing stays static while the loop is only partly unrolled.
#pragma unroll 2
        for (int w = 0; w < 8; ++w) {
            const uint32_t d = kw[0];
#pragma unroll
            for (int i = 0; i < 7; ++i) kw[i] = kw[i + 1];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float* e = table + ((4 * w + k) * E + ((d >> (8 * k)) & 0xffu)) * GP;
                if constexpr (GP == 4) {
                    const float4 x = *(const float4*)e;
                    sc[0] += x.x;
                    if (G > 1) sc[1 % G] += x.y;
                    if (G > 2) sc[2 % G] += x.z;
                    if (G > 3) sc[3 % G] += x.w;
                } else if constexpr (GP == 2) {
                    const float2 x = *(const float2*)e;
                    sc[0] += x.x;
                    sc[1 % G] += x.y;
                } else {
                    sc[0] += e[0];
                }
            }
        }
        if (t >= t_end) {
#pragma unroll
            for (int g = 0; g < G; ++g) sc[g] = kNegInf;
        }
        float p[G];
        softmax_tile<G, 4>(sc, m, l, acc, p);
#pragma unroll
        for (int g = 0; g < G; ++g) pw[lane * GP + g] = p[g];
        wave_lds_sync();
#pragma unroll 2
        for (int w = 0; w < 8; ++w) {
            const uint32_t d = vw[0];
#pragma unroll
            for (int i = 0; i < 7; ++i) vw[i] = vw[i + 1];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float* pp = pw + (half * 32 + 4 * w + k) * GP;
                float pv[G];
                if constexpr (GP == 4) {
                    const float4 x = *(const float4*)pp;
                    pv[0] = x.x;
                    if (G > 1) pv[1 % G] = x.y;
                    if (G > 2) pv[2 % G] = x.z;
                    if (G > 3) pv[3 % G] = x.w;
                } else {
#pragma unroll
                    for (int g = 0; g < G; ++g) pv[g] = pp[g];
                }
                const uint2 c = vbook[(d >> (8 * k)) & 0xffu];
                const float x0 = lo_half(c.x), x1 = hi_half(c.x), x2 = lo_half(c.y), x3 = hi_half(c.y);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    acc[g][0] += pv[g] * x0;
                    acc[g][1] += pv[g] * x1;
                    acc[g][2] += pv[g] * x2;
                    acc[g][3] += pv[g] * x3;
                }
            }
        }
        wave_lds_sync();
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = wave_sum(l[g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] += xor_lane(acc[g][i], 32);
    }
    __syncthreads();
    merge_and_store<G, 4, NW>(table, m, l, acc, a, b, h, s);
}

// ------------------------------------------------------------------ gather path

template <int FMT, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_gather_kernel(DecodeArgs a) {
    using F = DFmt<FMT>;
    constexpr int E = F::E, DS = F::DS, J = F::J, W = F::W;
    constexpr int NG = 64 / J;                              // token groups in the value mapping
    constexpr int TPG = 64 / NG;                            // tokens per group
    constexpr int BOOK_BYTES = E * DS * 2;
    constexpr int MERGE_BYTES = NW * G * (kHeadDim + 2) * 4;
    constexpr int A_BYTES = BOOK_BYTES > MERGE_BYTES ? BOOK_BYTES : MERGE_BYTES;
    __shared__ __align__(16) unsigned char region_a[A_BYTES];      // K book, then merge scratch
    __shared__ __align__(16) uint16_t vbook[E * DS];
    __shared__ __align__(16) float qs[G * kHeadDim];
    __shared__ __align__(16) float pbuf[NW][64 * G];
    uint16_t* kbook = (uint16_t*)region_a;

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t_begin = s * a.chunk;
    const int t_end = min(a.seq_len, t_begin + a.chunk);

    {
        const uint4* kb = (const uint4*)(a.k_book + (int64_t)h * E * DS);
        const uint4* vb = (const uint4*)(a.v_book + (int64_t)h * E * DS);
        for (int i = threadIdx.x; i < E * DS / 8; i += NW * 64) {
            ((uint4*)kbook)[i] = kb[i];
            ((uint4*)vbook)[i] = vb[i];
        }
        const float* qp = a.q_prime + ((int64_t)b * a.hq + h * G) * kHeadDim;
        for (int i = threadIdx.x; i < G * kHeadDim; i += NW * 64) qs[i] = qp[i] * a.qscale;
    }
    __syncthreads();

    float m[G], l[G], acc[G][DS];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
#pragma unroll
        for (int i = 0; i < DS; ++i) acc[g][i] = 0.0f;
    }
    const int64_t stream = (int64_t)b * a.hkv + h;
    const uint8_t* kbase = a.k_codes + stream * (int64_t)a.cap * W;
    const uint8_t* vbase = a.v_codes + stream * (int64_t)a.cap * W;
    const int jv = lane % J, grp = lane / J;
    float* pw = pbuf[wave];

    for (int tile = t_begin + wave * 64; tile < t_end; tile += NW * 64) {
        const int t = tile + lane;
        // Key codes of this lane's token, value codes of row jv of this lane's group.
        uint32_t kw[W / 4], vw[TPG * (FMT == 0 ? 1 : 3) / (FMT == 0 ? 1 : 2) / 4];
        if constexpr (FMT == 0) {
            const uint4* kc = (const uint4*)(kbase + (int64_t)t * 32);
            const uint4 k0 = kc[0], k1 = kc[1];
            kw[0] = k0.x; kw[1] = k0.y; kw[2] = k0.z; kw[3] = k0.w;
            kw[4] = k1.x; kw[5] = k1.y; kw[6] = k1.z; kw[7] = k1.w;
            const uint4* vc = (const uint4*)(vbase + (int64_t)(tile + grp * 32) * 32 + jv * 32);
            const uint4 v0 = vc[0], v1 = vc[1];
            vw[0] = v0.x; vw[1] = v0.y; vw[2] = v0.z; vw[3] = v0.w;
            vw[4] = v1.x; vw[5] = v1.y; vw[6] = v1.z; vw[7] = v1.w;
        } else {
            const uint2* kc = (const uint2*)(kbase + (int64_t)t * 24);
            const uint2 k0 = kc[0], k1 = kc[1], k2 = kc[2];
            kw[0] = k0.x; kw[1] = k0.y; kw[2] = k1.x; kw[3] = k1.y; kw[4] = k2.x; kw[5] = k2.y;
            const uint2* vc = (const uint2*)(vbase + (int64_t)(tile + grp * 16) * 24 + jv * 24);
            const uint2 v0 = vc[0], v1 = vc[1], v2 = vc[2];
            vw[0] = v0.x; vw[1] = v0.y; vw[2] = v1.x; vw[3] = v1.y; vw[4] = v2.x; vw[5] = v2.y;
        }
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = 0.0f;
        // Codes are consumed RW dwords (SUB sub-vectors) per step from the front
        // of a rotating window: static register indexing, bounded loads in flight.
        constexpr int RW = FMT == 0 ? 1 : 3, SUB = FMT == 0 ? 4 : 8;
#pragma unroll 1
        for (int j0 = 0; j0 < J; j0 += SUB) {
            uint32_t cw[RW];
#pragma unroll
            for (int i = 0; i < RW; ++i) cw[i] = kw[i];
#pragma unroll
            for (int i = 0; i < W / 4 - RW; ++i) kw[i] = kw[i + RW];
#pragma unroll
          for (int jj = 0; jj < SUB; ++jj) {
            const int j = j0 + jj;
            const uint32_t code = FMT == 0 ? byte_at(cw, jj) : code12_at(cw, jj);
            float c[DS];
            if constexpr (DS == 4) {
                const uint2 w = *(const uint2*)(kbook + code * 4);
                c[0] = lo_half(w.x); c[1] = hi_half(w.x); c[2] = lo_half(w.y); c[3] = hi_half(w.y);
            } else {
                const uint4 w = *(const uint4*)(kbook + code * 8);
                c[0] = lo_half(w.x); c[1] = hi_half(w.x); c[2] = lo_half(w.y); c[3] = hi_half(w.y);
                c[4] = lo_half(w.z); c[5] = hi_half(w.z); c[6] = lo_half(w.w); c[7] = hi_half(w.w);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float* q = qs + g * kHeadDim + j * DS;
#pragma unroll
                for (int i = 0; i < DS; ++i) sc[g] += q[i] * c[i];
            }
          }
        }
        if (t >= t_end) {
#pragma unroll
            for (int g = 0; g < G; ++g) sc[g] = kNegInf;
        }
        float p[G];
        softmax_tile<G, DS>(sc, m, l, acc, p);
#pragma unroll
        for (int g = 0; g < G; ++g) pw[lane * G + g] = p[g];
        wave_lds_sync();
        constexpr int VW = TPG * (FMT == 0 ? 1 : 3) / (FMT == 0 ? 1 : 2) / 4;
#pragma unroll 1
        for (int t0 = 0; t0 < TPG; t0 += SUB) {
            uint32_t cw[RW];
#pragma unroll
            for (int i = 0; i < RW; ++i) cw[i] = vw[i];
#pragma unroll
            for (int i = 0; i < VW - RW; ++i) vw[i] = vw[i + RW];
#pragma unroll
          for (int ti = 0; ti < SUB; ++ti) {
            const int tt = t0 + ti;
            const float* pp = pw + (grp * TPG + tt) * G;
            const uint32_t code = FMT == 0 ? byte_at(cw, ti) : code12_at(cw, ti);
            float c[DS];
            if constexpr (DS == 4) {
                const uint2 w = *(const uint2*)(vbook + code * 4);
                c[0] = lo_half(w.x); c[1] = hi_half(w.x); c[2] = lo_half(w.y); c[3] = hi_half(w.y);
            } else {
                const uint4 w = *(const uint4*)(vbook + code * 8);
                c[0] = lo_half(w.x); c[1] = hi_half(w.x); c[2] = lo_half(w.y); c[3] = hi_half(w.y);
                c[4] = lo_half(w.z); c[5] = hi_half(w.z); c[6] = lo_half(w.w); c[7] = hi_half(w.w);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pv = pp[g];
#pragma unroll
                for (int i = 0; i < DS; ++i) acc[g][i] += pv * c[i];
            }
          }
        }
        wave_lds_sync();
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = wave_sum(l[g]);
#pragma unroll
        for (int i = 0; i < DS; ++i) {
            if (NG >= 4) acc[g][i] += xor_lane(acc[g][i], 16);
            acc[g][i] += xor_lane(acc[g][i], 32);
        }
    }
    __syncthreads();
    merge_and_store<G, DS, NW>((float*)region_a, m, l, acc, a, b, h, s);
}

// ----------------------------------------------------------------------- combine

__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
    const int64_t bg = blockIdx.x;
    const int d = threadIdx.x;
    const float* lse = a.part_lse + bg * a.splits;
    float M = kNegInf;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, lse[s]);
    float num = 0.0f, den = 0.0f;
    if (M != kNegInf) {
        for (int s = 0; s < a.splits; ++s) {
            const float ls = lse[s];
            if (ls == kNegInf) continue;
            const float w = __builtin_amdgcn_exp2f(ls - M);
            den += w;
            num += w * a.part_o[(bg * a.splits + s) * kHeadDim + d];
        }
    }
    a.out[bg * kHeadDim + d] = den > 0.0f ? num / den : 0.0f;
}

template <int FMT, int NW>
hipError_t launch_gather(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    const int G = a.hq / a.hkv;
    switch (G) {
#define VQKV_G(GV) case GV: hipLaunchKernelGGL((decode_gather_kernel<FMT, GV, NW>), grid, dim3(NW * 64), 0, stream, a); break;
        VQKV_G(1) VQKV_G(2) VQKV_G(3) VQKV_G(4) VQKV_G(5) VQKV_G(6) VQKV_G(7) VQKV_G(8)
#undef VQKV_G
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid(a.splits, a.hkv, a.batch);
    const int G = a.hq / a.hkv;
    const bool table_ok = a.fmt == 0 && G <= 4;
    const bool use_table = table_ok && a.path != 2;
    if (a.path == 1 && !table_ok) return hipErrorInvalidValue;
    if (use_table) {
        constexpr int NW = 16;
        switch (G) {
            case 1: hipLaunchKernelGGL((decode_table_kernel<1, NW>), grid, dim3(NW * 64), 0, stream, a); break;
            case 2: hipLaunchKernelGGL((decode_table_kernel<2, NW>), grid, dim3(NW * 64), 0, stream, a); break;
            case 3: hipLaunchKernelGGL((decode_table_kernel<3, NW>), grid, dim3(NW * 64), 0, stream, a); break;
            case 4: hipLaunchKernelGGL((decode_table_kernel<4, NW>), grid, dim3(NW * 64), 0, stream, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.fmt == 0) return launch_gather<0, 8>(a, grid, stream);
    return launch_gather<1, 8>(a, grid, stream);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(combine_kernel, dim3(a.batch * a.hq), dim3(128), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vqkv
