// attn_common.h -- online-softmax and split-merge steps shared by the decode kernels.
#pragma once

#include "device_util.h"
#include "internal.h"
#include "qtransform.h"

namespace vqkv {

constexpr float kNegInf = -__builtin_inff();

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

// The same update for tiles whose scores rarely raise the running max: a
// ballot checks whether any lane exceeds it, and only then are the tile
// maxima reduced across the wave and the state rescaled (rescale(g, alpha)
// multiplies head g's sum l and output accumulators by alpha).  p comes out
// multiplied by 2^P_LOG2 (the caller's fixed scale for l and the accumulators).
template <int G, int P_LOG2, class Rescale>
__device__ __forceinline__ void softmax_tile_lazy(float (&sc)[G], float (&m)[G], float (&p)[G],
                                                  Rescale&& rescale) {
    bool up = false;
#pragma unroll
    for (int g = 0; g < G; ++g) up = up || (sc[g] > m[g]);
    if (__ballot(up)) {                                     // wave-uniform
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mn = fmaxf(m[g], wave_max(sc[g]));
            if (mn != m[g]) {
                rescale(g, __builtin_amdgcn_exp2f(m[g] - mn));
                m[g] = mn;
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) p[g] = __builtin_amdgcn_exp2f(sc[g] - m[g] + (float)P_LOG2);
}

// softmax_tile_lazy for scores that arrive scaled: head g's scores (and m[g],
// kept in the same units) are its true scores times 2^-k_g, and sm[g] = 2^k_g
// takes them back inside the exponents.  With sm[g] = 1 every result is
// bit-identical to softmax_tile_lazy (x * 1 is exact and the fused add rounds
// once, as the plain add does).
template <int G, int P_LOG2, class Rescale>
__device__ __forceinline__ void softmax_tile_lazy_scaled(float (&sc)[G], float (&m)[G], const float (&sm)[G],
                                                         float (&p)[G], Rescale&& rescale) {
    bool up = false;
#pragma unroll
    for (int g = 0; g < G; ++g) up = up || (sc[g] > m[g]);
    if (__ballot(up)) {                                     // wave-uniform
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mn = fmaxf(m[g], wave_max(sc[g]));
            if (mn != m[g]) {
                rescale(g, __builtin_amdgcn_exp2f((m[g] - mn) * sm[g]));
                m[g] = mn;
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) p[g] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[g] - m[g], sm[g], (float)P_LOG2));
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi, a and b holding fp16 pairs; fp32 accumulate.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// (lo, hi) -> fp16 pair, round to nearest even (one v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    const half2_t h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}

// Merge the NW waves' states and write the split's partial: its normalized
// output o and the pair (m, ll), m the largest score and ll = log2 of the
// sum of 2^(z - m) over the split's tokens (log-sum-exp = m + ll, kept as two
// numbers so the merge of splits stays exact whatever the size of m).
// `scratch` holds, per wave w and head g, the unnormalized output at
// scratch[(w * G + g) * 128 + d] and (m, l) at scratch[NW * G * 128 +
// (w * G + g) * 2 + {0, 1}]; every thread of the block calls this after a
// barrier.  l_log2_scale is a power-of-two factor carried by l and the
// outputs (removed from ll).
template <int G, int NW>
__device__ __forceinline__ void merge_waves(const float* scratch, const DecodeArgs& a, int b, int h, int s,
                                            float l_log2_scale, float* stage = nullptr) {
    const float* mo = scratch;
    const float* ml = scratch + NW * G * kHeadDim;
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += NW * 64) {
        const int g = idx / kHeadDim, d = idx % kHeadDim;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ml[(w * G + g) * 2]);
        float o = 0.0f, ll = 0.0f;
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
            ll = __builtin_log2f(L) - l_log2_scale;
        }
        if (stage != nullptr && a.out != nullptr && (a.splits > 1 || a.v_smooth != nullptr)) {
            // Fused combine (the partial waits in LDS for combine_if_last), or one
            // split of the value-transform variant (o waits for its output map).
            stage[g * kHeadDim + d] = o;
            if (d == 0) {
                stage[G * kHeadDim + 2 * g] = M;
                stage[G * kHeadDim + 2 * g + 1] = ll;
            }
        } else if (a.out != nullptr && a.splits == 1) {
            // One split: o is already the output (the combine of a single
            // split returns it unchanged, 0 for an empty row).
            a.out[((int64_t)b * a.hq + h * G + g) * kHeadDim + d] = o;
        } else {
            const int64_t row = ((int64_t)b * a.hq + h * G + g) * a.splits + s;
            a.part_o[row * kHeadDim + d] = o;
            if (d == 0) {
                a.part_ml[2 * row] = M;
                a.part_ml[2 * row + 1] = ll;
            }
        }
    }
}

// One (b, q-head) row of the split combine: with M the largest m_i,
// x_i = (m_i - M) + ll_i and X the largest x_i, out = sum_i w_i o_i / sum_i
// w_i, w_i = 2^(x_i - X) (empty splits, m_i = -inf, weigh 0; a row with no
// token gives 0).  m_i - M is exact wherever it decides a weight (m_i within a
// factor 2 of M), so the weights keep full precision at any score size, and
// the heaviest split weighs exactly 1 (one split returns its o unchanged).
// d = output dim in [0, 128) of the row's 128-thread
// group; red = 2 floats and wts = 128 floats of LDS for the group.  Splits go
// in chunks of 128: thread d computes the weight of split c + d into wts, then
// every thread sums its dim over the chunk in split order, 16 partial rows in
// flight.  It has block barriers: every thread of the block calls it, threads
// of an inactive group only pass the barriers.
__device__ __forceinline__ void combine_row(const float* part_o, const float* part_ml, float* out, int S,
                                            int64_t bg, int d, bool active, float* red, float* wts,
                                            float* lds_row = nullptr) {
    const int lane = d & 63, wave = d >> 6;
    const float* ml = part_ml + bg * S * 2;
    float M = kNegInf;
    if (active)
        for (int s = d; s < S; s += 128) M = fmaxf(M, ml[2 * s]);
    M = wave_max(M);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = fmaxf(red[0], red[1]);
    __syncthreads();
    const bool any = active && M != kNegInf;
    float X = kNegInf;
    if (any)
        for (int s = d; s < S; s += 128)
            if (ml[2 * s] != kNegInf) X = fmaxf(X, (ml[2 * s] - M) + ml[2 * s + 1]);
    X = wave_max(X);
    if (lane == 0) red[wave] = X;
    __syncthreads();
    X = fmaxf(red[0], red[1]);
    __syncthreads();
    const float* po = part_o + bg * S * kHeadDim + d;
    float den = 0.0f, num = 0.0f;
    for (int c = 0; c < S; c += 128) {                      // the same trip count in every thread
        float w = 0.0f;
        if (any && c + d < S) {
            const float ms = ml[2 * (c + d)];
            w = ms == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(((ms - M) + ml[2 * (c + d) + 1]) - X);
        }
        den += w;
        wts[d] = w;
        __syncthreads();
        if (any) {
            const int n = S - c < 128 ? S - c : 128;
#pragma unroll 16
            for (int i = 0; i < n; ++i) num += wts[i] * po[(int64_t)(c + i) * kHeadDim];
        }
        __syncthreads();
    }
    den = wave_sum(den);
    if (lane == 0) red[wave] = den;
    __syncthreads();
    den = red[0] + red[1];
    const float r = den > 0.0f ? num / den : 0.0f;
    if (active) {
        if (lds_row != nullptr) lds_row[d] = r;            // the caller maps the row back
        else out[bg * kHeadDim + d] = r;
    }
}

// Fused combine after merge_waves(..., stage), for more than one split.
// Wave 0 writes the split's partials (G rows of o, G (m, ll) pairs, staged in
// LDS by merge_waves), makes them visible device-wide with one release fence,
// and counts the work-group in arrivals[b][h] (lane 0, after the fence: all of
// the wave's stores precede the count).  The last of the head's splits to
// arrive fences again (acquire) before the block reads the other splits'
// partials, combines the head's G rows (one 128-thread group per query head)
// and clears the counter for the next launch.  One fence pair per work-group:
// a device-scope fence writes back the L2 of the XCD, too slow to run in every
// wave.
template <int G, int NW>
__device__ __forceinline__ void combine_if_last(unsigned char* smem, const float* stage, const DecodeArgs& a,
                                                int b, int h) {
    static_assert(G * 128 <= NW * 64, "one 128-thread group per query head");
    int* last = (int*)smem;
    float* red = (float*)(smem + 16);                       // 2 floats per group
    float* wts = (float*)(smem + 128);                      // 128 floats per group
    const int64_t stream = (int64_t)b * a.hkv + h;
    __syncthreads();                                        // the stage is complete, the merge scratch free
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x, s = blockIdx.x;
        for (int i = lane; i < G * kHeadDim; i += 64) {
            const int64_t row = ((int64_t)b * a.hq + h * G + i / kHeadDim) * a.splits + s;
            a.part_o[row * kHeadDim + i % kHeadDim] = stage[i];
        }
        if (lane < 2 * G)
            a.part_ml[2 * (((int64_t)b * a.hq + h * G + lane / 2) * a.splits + s) + lane % 2] = stage[G * kHeadDim + lane];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        int prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(a.arrivals + stream, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __shfl(prev, 0, 64);
        if (prev == a.splits - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0) *last = prev == a.splits - 1;
    }
    __syncthreads();
    if (!*last) return;                                     // block-uniform
    const int grp = threadIdx.x >> 7;
    const bool active = grp < G;
    // Value-transform variant: the combined rows wait in LDS for the output map.
    float* rows = a.v_smooth != nullptr ? (float*)(smem + 4352) : nullptr;   // G x 128 floats
    combine_row(a.part_o, a.part_ml, a.out, a.splits, (int64_t)b * a.hq + h * G + (active ? grp : 0),
                threadIdx.x & 127, active, red + 2 * grp, wts + 128 * grp, rows ? rows + 128 * grp : nullptr);
    if (rows != nullptr) {                                  // block-uniform
        __syncthreads();
        const int wave = threadIdx.x >> 6;
        if (wave < G)
            value_untransform_wave(rows + 128 * wave, a.v_smooth + (int64_t)h * kHeadDim,
                                   a.out + ((int64_t)b * a.hq + h * G + wave) * kHeadDim, threadIdx.x & 63);
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.arrivals + stream, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stash one wave's (m, l) for merge_waves (lane 0 writes).
template <int G, int NW>
__device__ __forceinline__ void stash_ml(float* scratch, const float (&m)[G], const float (&l)[G]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float* ml = scratch + NW * G * kHeadDim;
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ml[(wave * G + g) * 2] = m[g];
            ml[(wave * G + g) * 2 + 1] = l[g];
        }
    }
}

// Stash and merge for accumulators laid out as lanes [0, 128 / DS) of each
// wave holding dims [lane * DS, lane * DS + DS) (already token-group reduced).
// `scratch` must hold NW * G * (128 + 2) floats and be free for reuse (the
// caller synchronizes before).
template <int G, int DS, int NW>
__device__ __forceinline__ void merge_and_store(float* scratch, const float (&m)[G], const float (&l)[G],
                                                const float (&acc)[G][DS], const DecodeArgs& a,
                                                int b, int h, int s, float l_log2_scale = 0.0f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane < kHeadDim / DS) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < DS; ++i) scratch[(wave * G + g) * kHeadDim + lane * DS + i] = acc[g][i];
    }
    stash_ml<G, NW>(scratch, m, l);
    __syncthreads();
    merge_waves<G, NW>(scratch, a, b, h, s, l_log2_scale);
}

}  // namespace vqkv
