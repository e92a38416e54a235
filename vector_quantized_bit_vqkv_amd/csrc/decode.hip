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
// (o normalized, m, ll) to the workspace: m the largest score, ll the log2 of
// the weight sum, so the log-sum-exp is m + ll.  Scores carry the factor
// sm_scale * log2(e), so exp2 is the exponential and m, ll are in log2 units.
//
// Kernels (the matrix-core one chosen by measurement; the others stay
// selectable for measurement):
//   * decode_mfma_kernel (default, every format: 2-bit 2^8 x 4, 1.5-bit
//     2^12 x 8, 3-bit 2^12 x 4, 1.25-bit 2^10 x 8, 4-bit 2^8 x 2): scores
//     and values both on the matrix cores,
//     v_mfma_f32_4x4x4f16, with the centroids gathered from LDS codebooks
//     (details at the kernel).  For the fused decode step it also finishes
//     the output: with one split the work-group writes it directly, with more
//     the last split of a head to finish combines the head's splits, and in
//     the value-transform variant the output is mapped back, s_v * (H o);
//   * decode_table_kernel (2-bit, G <= 4): per work-group score table
//     L[j][e][g] = c * q'_g[4j..4j+3] . C_K[e] for all 32 x 256 (j, e), so a
//     token's score is 32 table reads and adds; values on the matrix cores;
//   * decode_gather_kernel (2-bit and 1.5-bit): the token's centroids are read
//     from the LDS codebook and dotted with q' (held in LDS, pre-scaled).
#include "attn_common.h"
#include "device_util.h"
#include "internal.h"
#include "qtransform.h"
#include "token_search.h"

// Every instantiation evaluates each expression the same way (no fused
// multiply-add formed by the compiler), so the contiguous, paged, ragged and
// fused-step forms of a kernel give bit-identical results by construction.
#pragma clang fp contract(off)

namespace vqkv {

namespace {

// Context length of sequence b: the uniform seq_len, or the caller's
// per-sequence length clamped to [0, capacity] (an out-of-range length can
// never make a kernel read outside the cache).
__device__ __forceinline__ int seq_len_of(const DecodeArgs& a, int b) {
    if (a.seq_lens) {
        const int n = a.seq_lens[b];
        return n < 0 ? 0 : (n > a.cap ? a.cap : n);
    }
    if (a.app.positions) {                                  // fused append: through the new token
        const int64_t p = a.app.positions[b];
        return p < 0 ? 0 : (p >= a.cap ? a.cap : (int)p + 1);
    }
    return a.seq_len;
}

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

// ------------------------------------------------------------ score-table path

// Score table layout.  Entry (j, e) holds the four heads' fixed-point scores
// (16 bytes).  Rows are indexed by the code e: half h = j / 16 of the table is
// [256 codes][16 columns][16 B], so a row is 256 bytes and column j % 16 sits
// in bank group j % 16.  At step s lane l reads sub-vector j = s ^ (l % 16):
// the 16 lanes of each 16-byte-read pass then touch 16 different bank groups
// whatever their codes are (no bank conflicts), and the address is a byte
// permutation: code -> byte 1, column * 16 -> byte 0, half -> byte 2.
constexpr int kTabHalfBytes = 256 * 16 * 16;

// b in the lanes whose bit is set in `mask`, a elsewhere.
__device__ __forceinline__ uint32_t lane_select(uint32_t a, uint32_t b, uint64_t mask) {
    uint32_t d;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(mask));
    return d;
}
// ------------------------------------------------------ values on the matrix cores
//
// The value product o_g += sum_t p_{g,t} * C_V[vc_{t,j}] of a 64-token tile
// runs on v_mfma_f32_4x4x4f16: 16 independent 4x4x4 products per wave, block
// b = lane / 4, A row i in lane 4b + i, B column j in lane 4b + j, result
// D[i][j] in register i of lane 4b + j.  Per step of 4 tokens and per half of
// the sub-vectors (16 of them, 64 dims): A = the probabilities (row i = head
// i, the same in every block) and B of block b = the 4 tokens' dims of
// sub-vector 16*half + b.  B comes straight from the codebook in LDS through
// the transposing read ds_read_b64_tr_b16, where lane 16r + i receives
// element i % 4 of the 8-byte rows addressed by lanes 16r + 4e + i / 4, as
// its elements e = 0..3.  So lane 16r + 4k + q looks up the centroid of the
// step's token k for sub-vector 16*half + 4r + q, and block b = 4r + q
// receives exactly its (token, dim) operand.  Lane L ends up accumulating
// dims L and 64 + L of every head.  The value-code layout gives each lane one
// 32-byte chunk per tile: byte 2s + half is its lookup for step s.

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ half4_t lds_read_tr16(const lds_char* p) {
    return __builtin_bit_cast(half4_t,
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(lds_char*)p));
}

__device__ __forceinline__ float4_t mfma_4x4x4(half4_t a, half4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0);
}

// Store this lane's fp16 probabilities (scaled, G heads) into the wave's
// A-operand buffer: step s (tokens 4s..4s+3) takes 8 * HB dwords, head g's
// four tokens in dwords 2g and 2g + 1.  Even lanes write the pair (t, t+1).
// l accumulates the same rounded pairs; every lane adds its pair (the odd lane
// in swapped order), so l counts each token twice.
template <int G, int HB>
__device__ __forceinline__ void store_probs(uint32_t* pw, const float (&p)[G], float (&l)[G], int lane) {
    constexpr uint32_t kOnes = 0x3c003c00u;                 // (1.0, 1.0) in fp16
    uint32_t pkp[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        pkp[g] = pack_half2(p[g], dpp<0xB1>(p[g]));
        l[g] = dot2(pkp[g], kOnes, l[g]);
    }
    if (!(lane & 1)) {
        uint32_t* dst = pw + (lane >> 2) * (8 * HB) + ((lane >> 1) & 1);
#pragma unroll
        for (int g = 0; g < G; ++g) dst[2 * g] = pkp[g];
    }
}

// Value codebook: 8 copies, copy c of entry e at e * 64 + c * 8; lane l uses
// copy l % 8, which spreads a pass of 32 lanes over all 32 bank pairs.
constexpr int kVCopies = 8;

template <int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_table_kernel(DecodeArgs a) {
    static_assert(G >= 1 && G <= 4, "score table holds four heads");
    constexpr int E = 256;
    __shared__ __align__(16) int32_t table[2 * kTabHalfBytes / 4];
    __shared__ __align__(16) uint2 vrep[E * kVCopies];
    __shared__ __align__(16) uint32_t pbuf[NW][16 * 8];   // fp16 probabilities, [step][head][4 tokens]
    __shared__ float wmax[NW];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t_begin = s * a.chunk;
    const int t_end = min(seq_len_of(a, b), t_begin + a.chunk);

    {
        const uint2* vb = (const uint2*)(a.v_book + (int64_t)h * E * 4);
        for (int i = threadIdx.x; i < E * kVCopies; i += NW * 64) vrep[i] = vb[i / kVCopies];
        // Rows of heads >= G stay zero (their products are computed and dropped).
        for (int i = threadIdx.x; i < NW * 16 * 8; i += NW * 64) (&pbuf[0][0])[i] = 0u;
    }
    // Build the table in fp32, find max |L|, then convert in place to int32
    // round(L * 2^F) with 2^F * max|L| <= 2^26 (32 entries cannot overflow).
    float* tablef = (float*)table;
    float lmax = 0.0f;
    {
        const uint2* kb = (const uint2*)(a.k_book + (int64_t)h * E * 4);
        const float* qp = a.q_prime + ((int64_t)b * a.hq + h * G) * kHeadDim;
        for (int idx = threadIdx.x; idx < 32 * E; idx += NW * 64) {
            const int e = idx & 255, j = idx >> 8;
            const uint2 c = kb[e];
            const float c0 = lo_half(c.x), c1 = hi_half(c.x), c2 = lo_half(c.y), c3 = hi_half(c.y);
            float v[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                v[g] = 0.0f;
                if (g < G) {
                    const float4 q = *(const float4*)(qp + g * kHeadDim + 4 * j);
                    v[g] = (q.x * c0 + q.y * c1 + q.z * c2 + q.w * c3) * a.qscale;
                }
                lmax = fmaxf(lmax, fabsf(v[g]));
            }
            const int off = (j >> 4) * kTabHalfBytes + e * 256 + (j & 15) * 16;
            *(float4*)((char*)tablef + off) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
    lmax = wave_max(lmax);
    if (lane == 0) wmax[wave] = lmax;
    __syncthreads();
    lmax = wmax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) lmax = fmaxf(lmax, wmax[w]);
    int fexp = 26;
    if (lmax > 0.0f) {
        int ex;
        frexpf(lmax, &ex);                                  // lmax < 2^ex
        fexp = 26 - ex;
    }
    const float to_fixed = __builtin_ldexpf(1.0f, fexp);
    const float from_fixed = __builtin_ldexpf(1.0f, -fexp);
    for (int i = threadIdx.x; i < 2 * kTabHalfBytes / 4; i += NW * 64)
        table[i] = (int32_t)__builtin_rintf(tablef[i] * to_fixed);
    __syncthreads();

    float m[G], l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
    }
    float4_t o[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    const int64_t stream = (int64_t)b * a.hkv + h;
    const uint8_t* kbase = a.k_codes + stream * (int64_t)a.cap * 32;
    const uint8_t* vbase = a.v_codes + stream * (int64_t)a.cap * 32;
    uint32_t* pw = pbuf[wave];
    const char* pa_base = (const char*)pw + (lane & 3) * 8;
    const lds_char* vt = (const lds_char*)vrep;
    // Lane constants of the conflict-free table walk.
    const uint32_t lam = lane & 15;
    const uint32_t lam3 = lam & 3;
    const uint32_t byte_sel = (0u ^ lam3) | ((1u ^ lam3) << 8) | ((2u ^ lam3) << 16) | ((3u ^ lam3) << 24);
    const uint32_t lx = lam << 4;
    const uint32_t vslot = (lane & (kVCopies - 1)) * 8;
    // p is produced as exp2(score - max + 15): the fp16 pairs then stay clear of
    // the subnormal range down to 2^-29 of the maximum.  l and acc carry the
    // same 2^15, removed from ll at the end.
    constexpr int P_LOG2 = 15;
    const char* tab = (const char*)table;

    // Each code register is reloaded with the next tile's codes right after its
    // last use in this tile: key codes once they are permuted (a whole tile of
    // work hides the latency), value codes one 16-byte half at a time during
    // the value phase.  No second buffer and no copies; the next tile index is
    // clamped to a valid tile so the loads are unconditional and in bounds.
    constexpr int kStride = NW * 64;
    const int first = t_begin + wave * 64;
    const uint4* kc0 = (const uint4*)(kbase + (int64_t)lane * 32);
    const uint4* vc0 = (const uint4*)(vbase + (int64_t)lane * 32);
    uint4 ck0, ck1, cv0, cv1;
    if (first < t_end) {
        ck0 = kc0[(int64_t)first * 2];
        ck1 = kc0[(int64_t)first * 2 + 1];
        cv0 = vc0[(int64_t)first * 2];
        cv1 = vc0[(int64_t)first * 2 + 1];
    }

    for (int tile = first; tile < t_end; tile += kStride) {
        const int t = tile + lane;
        const int nxt = tile + kStride < t_end ? tile + kStride : tile;
        uint32_t kw[8] = {ck0.x, ck0.y, ck0.z, ck0.w, ck1.x, ck1.y, ck1.z, ck1.w};
        // Permute the code bytes so that byte s holds sub-vector s ^ lam.
        uint32_t pk[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) pk[w] = __builtin_amdgcn_perm(0u, kw[w], byte_sel);
        {
            // Dword swaps by bits 2 and 3 of the lane index: fixed lane masks,
            // one v_cndmask per word and stage.
            uint32_t q[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) q[w] = lane_select(pk[w], pk[w ^ 1], 0xF0F0F0F0F0F0F0F0ull);
#pragma unroll
            for (int w = 0; w < 8; ++w) pk[w] = lane_select(q[w], q[w ^ 2], 0xFF00FF00FF00FF00ull);
        }
        __builtin_amdgcn_sched_barrier(0);
        ck0 = kc0[(int64_t)nxt * 2];
        ck1 = kc0[(int64_t)nxt * 2 + 1];
        // Scores, lane = token: 32 table reads, summed two at a time.
        int32_t si[4] = {0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < 32; st += 2) {
            int4 x[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int s2 = st + u;
                const uint32_t ofs = lx ^ ((uint32_t)((s2 & 15) << 4) | ((uint32_t)(s2 >> 4) << 16));
                const uint32_t sel = 0x0c020000u | ((4u + (uint32_t)(s2 & 3)) << 8);
                const uint32_t addr = __builtin_amdgcn_perm(pk[s2 >> 2], ofs, sel);
                x[u] = *(const int4*)(tab + addr);
            }
            si[0] += x[0].x + x[1].x;
            si[1] += x[0].y + x[1].y;
            si[2] += x[0].z + x[1].z;
            si[3] += x[0].w + x[1].w;
        }
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = t < t_end ? (float)si[g] * from_fixed : kNegInf;
        float p[G];
        softmax_tile_lazy<G, P_LOG2>(sc, m, p, [&](int g, float alpha) {
            l[g] *= alpha;
            o[0][g] *= alpha;
            o[1][g] *= alpha;
        });
        store_probs<G, 1>(pw, p, l, lane);
        wave_lds_sync();
        // Values on the matrix cores, 8 steps (one 16-byte code half) at a time.
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
            const uint4 cv = hv == 0 ? cv0 : cv1;
            const uint32_t vwh[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const half4_t pa = *(const half4_t*)(pa_base + (8 * hv + 2 * w + q) * 32);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const uint32_t code = (vwh[w] >> (16 * q + 8 * hh)) & 0xffu;
                        o[hh] = mfma_4x4x4(pa, lds_read_tr16(vt + ((code << 6) | vslot)), o[hh]);
                    }
                }
            }
            // Issue the reload only after the old codes' last use (no copies).
            __builtin_amdgcn_sched_barrier(0);
            if (hv == 0) cv0 = vc0[(int64_t)nxt * 2];
            else cv1 = vc0[(int64_t)nxt * 2 + 1];
        }
        wave_lds_sync();
    }

#pragma unroll
    for (int g = 0; g < G; ++g) l[g] = 0.5f * wave_sum(l[g]);
    __syncthreads();
    float* scratch = (float*)table;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        scratch[(wave * G + g) * kHeadDim + lane] = o[0][g];
        scratch[(wave * G + g) * kHeadDim + 64 + lane] = o[1][g];
    }
    stash_ml<G, NW>(scratch, m, l);
    __syncthreads();
    merge_waves<G, NW>(scratch, a, b, h, s, (float)P_LOG2);
}

// --------------------------------------------------------- matrix-core path (2-bit)
//
// Scores and values both on v_mfma_f32_4x4x4f16.  Scores, lane = token: block
// b holds tokens 4b..4b+3 (B = their centroids of one sub-vector, one plain
// 8-byte LDS read per lane) and A = the query dims of that sub-vector (row i =
// head i).  The A operands of all 32 sub-vectors live in two register pairs:
// with CBSZ = 4 the instruction broadcasts block ABID's A to all 16 blocks,
// so lane 4c + i keeps head i's dims of sub-vectors c and 16 + c.  The query
// enters as fp16 (round to nearest; relative error 2^-11, finer than the bf16
// query it comes from); products are exact and sums fp32.  The result lands
// as lane = token, register = head, the layout the online softmax works in.  The probabilities are then
// turned to lane 4s + i = head i's tokens 4s..4s+3 (one 8-byte LDS write and
// one transposing read) and broadcast as the A operand of step s of the value
// product described above.
//
// Codebooks sit at a 256-byte stride per code: 32 copies of each 8-byte
// centroid, lane l reading copy l % 32, so the 32 lanes of an LDS pass hit 32
// distinct bank pairs whatever their codes.  A lookup address is then one byte
// permutation: copy * 8 in byte 0, the code in byte 1, the book in byte 2.
constexpr int kBookStride = 256;
constexpr int kBookBytes = 256 * kBookStride;

// Fused append of the one-split decode step (2-bit).  The work-group of
// (b, h) writes q' = H (q * s) of its G query heads into qr (waves 4..3+G,
// the query transform's own butterflies), then codes the new key and value of
// (b, h) with the exact fp64 search of the one-token append kernel (the same
// functions, so the codes are identical) and stores them in the cache.  It
// ends on a barrier: every code the work-group reads afterwards, the new
// token's included, is in place (the stores and the later loads come from one
// work-group on one CU).  `books` holds the staged K and V books, 32 copies
// per entry (entry e, copy c at byte kBookStride e + 8 c), staged but not yet
// synchronized; xr is 2 x 128 doubles of LDS.
// What the fused append reads from global memory, fetched before the first
// tiles' code loads are issued: loads complete in order, so any wait for
// these would otherwise also wait for the codes.  t is the token's position
// (uniform; scalar loads), `app` whether it lies inside the cache.
struct AppendFetch {
    int64_t t;
    bool app;
    QueryPair qv;       // waves 4 .. 3 + G: the query row's elements and scales
    uint32_t e;         // threads < 256: the key (value) element, raw (bf16 or fp32 bits)
    float div;          // and its divisor
    bool has_div;
};

// Uniform reads through the constant address space become scalar loads (the
// arrays are not written by the kernel).
template <class T>
__device__ __forceinline__ T scalar_read(const T* p, int64_t i) {
    return ((const __attribute__((address_space(4))) T*)p)[i];
}

template <int G, int NW>
__device__ __forceinline__ AppendFetch fused_append_fetch(const DecodeArgs& a, int b, int h) {
    const AppendArgs& ap = a.app;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t stream = (int64_t)b * a.hkv + h;
    AppendFetch f;
    // Position of the token: uniform, or per sequence; outside the cache it is
    // not appended (block-uniform), as in the append kernel.  With several
    // splits only the work-group whose token range holds it appends it (the
    // others never read that tile); every work-group transforms the query.  A
    // position past the last split's range (a ragged step whose max_seq_len
    // is below positions[b] + 1: no split attends to it) is appended by the
    // last split, so the cache still receives it as the append call would.
    f.t = ap.positions ? (int64_t)scalar_read(ap.positions, b) : (int64_t)ap.start_pos;
    const int64_t t_begin = (int64_t)blockIdx.x * a.chunk;
    f.app = f.t >= 0 && f.t < a.cap && f.t >= t_begin &&
            (f.t < t_begin + a.chunk || blockIdx.x == gridDim.x - 1);
    f.qv = QueryPair{0u, 0u, 0.0f, 0.0f, ap.dtype};
    if (wave >= 4 && wave < 4 + G) {
        const int64_t vec = (int64_t)b * a.hq + h * G + (wave - 4);
        f.qv = load_query_pair((const char*)ap.q + vec * kHeadDim * (ap.dtype == 0 ? 2 : 4), ap.dtype,
                               ap.smooth + (int64_t)h * kHeadDim, lane);
    }
    {
        // Threads < 256: the key (value) element c and its divisor.  Every
        // thread loads (the others element 0 and scale 0, always present), so
        // no branch joins a loaded value with a constant: the compiler would
        // convert right after the load and wait for it there.
        const bool mine = f.app && threadIdx.x < 2 * kHeadDim;
        const int c = threadIdx.x & (kHeadDim - 1), isv = (threadIdx.x >> 7) & 1;
        // Keys, and values of the value-transform variant: divided by their scales.
        const float* div = isv ? a.v_smooth : ap.smooth;
        const void* row = isv ? ap.v_new : ap.k_new;
        const int64_t i = mine ? stream * kHeadDim + c : 0;
        f.e = ap.dtype == 0 ? (uint32_t)((const uint16_t*)row)[i] : ((const uint32_t*)row)[i];
        f.has_div = div != nullptr;
        f.div = (div ? div : ap.smooth)[mine ? (int64_t)h * kHeadDim + c : 0];
    }
    return f;
}

template <int G, int NW>
__device__ __forceinline__ void fused_append_2bit(const DecodeArgs& a, int b, int h, const AppendFetch& f,
                                                  double* xr, float* qr, const unsigned char* books,
                                                  double* wide) {
    static_assert(NW == 16 && 4 + G <= NW, "64 sub-vectors x 16 slices fill the 1024 threads");
    const AppendArgs& ap = a.app;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t stream = (int64_t)b * a.hkv + h;
    const int64_t t = f.t;
    const bool app = f.app;
    if (wave >= 4 && wave < 4 + G) transform_query_pair(f.qv, qr + (wave - 4) * kHeadDim, lane);
    if (app && threadIdx.x < 2 * kHeadDim) {
        const int c = threadIdx.x & (kHeadDim - 1), isv = threadIdx.x >> 7;
        // bf16 bits widen exactly (a select, so the conversion stays here).
        const double e = (double)__builtin_bit_cast(float, ap.dtype == 0 ? f.e << 16 : f.e);
        xr[isv * kHeadDim + c] = f.has_div ? e / (double)f.div : e;
    }
    __syncthreads();
    if (app && (wave == 0 || (wave == 1 && a.v_smooth != nullptr))) rotate_row_wave(xr + wave * kHeadDim, lane);
    if (app) {
        // Both books (copy 0 of the staged copies), widened to fp64 once: the
        // search then converts nothing (the conversions were two of every
        // five of its instructions).  Two elements per thread.
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = threadIdx.x + NW * 64 * r;        // element of [2][256][4]
            const int isv = i >> 10, e = (i >> 2) & 255, c = i & 3;
            wide[i] = (double)half_bits_to_float(
                ((const uint16_t*)(books + isv * kBookBytes + e * kBookStride))[c]);
        }
    }
    __syncthreads();
    if (app) {
        // Sub-vector sv = thread / 16: key j = sv for sv < 32, value j = sv - 32;
        // slice sl = entries sl, sl + 16, ..., copy lane % 32 of the book.
        const int sv = threadIdx.x >> 4, sl = threadIdx.x & 15;
        const int isv = sv >> 5, j = sv & 31;
        double xs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[i] = xr[isv * kHeadDim + 4 * j + i];
        const double* book = wide + isv * 1024;
        double best = __builtin_inf();
        int idx = sl;
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const int e = sl + 16 * k;
            const double d = dist_f64<4>(xs, book + 4 * e);
            if (d < best) { best = d; idx = e; }
        }
        group_argmin<16>(best, idx);
        // The token's 64-token block: in the stream, or (paged) the pool block
        // the table names, clamped to the pool (a uniform, scalar read).
        int64_t blk;
        if (ap.block_table) {
            int pb = scalar_read(ap.block_table, stream * (int64_t)(a.cap >> 6) + (t >> 6));
            pb = pb < 0 ? 0 : (pb >= ap.num_blocks ? ap.num_blocks - 1 : pb);
            blk = (int64_t)pb * 2048;
        } else {
            blk = stream * (int64_t)a.cap * 32 + (t >> 6) * 2048;
        }
        if (sl == 0) {
            const int u = (int)(t & 63);
            if (isv == 0) ap.k_codes[blk + u * 32 + j] = (uint8_t)idx;
            else ap.v_codes[blk + v_code_offset_2bit(u, j)] = (uint8_t)idx;
        }
    }
    __syncthreads();
}

template <int V> struct IntC { static constexpr int value = V; };

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(IntC<I>{});
        static_for<I + 1, N>(f);
    }
}

template <int ABID>
__device__ __forceinline__ float4_t mfma_bcast(half4_t a, half4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}

// Selector of v_perm_b32(word, ofs, sel): byte 0 and 2 from ofs, byte 1 =
// byte k of word, byte 3 = 0.
template <int K>
constexpr uint32_t lookup_sel() { return 0x0c020000u | ((4u + K) << 8); }

// 24-bit little-endian value of bytes B..B+2 of a dword array (one v_perm_b32).
template <int B, int N>
__device__ __forceinline__ uint32_t bytes3_at(const uint32_t (&w)[N]) {
    constexpr int d = B >> 2;
    constexpr int d1 = (B + 2) >> 2;
    constexpr uint32_t s0 = ((B + 0) >> 2) == d ? ((B + 0) & 3) : 4 + ((B + 0) & 3);
    constexpr uint32_t s1 = ((B + 1) >> 2) == d ? ((B + 1) & 3) : 4 + ((B + 1) & 3);
    constexpr uint32_t s2 = ((B + 2) >> 2) == d ? ((B + 2) & 3) : 4 + ((B + 2) & 3);
    return __builtin_amdgcn_perm(w[d1], w[d], s0 | (s1 << 8) | (s2 << 16) | (0x0cu << 24));
}

// 2^SH x the BITS-bit code at bits [BITS C, BITS C + BITS) of the
// little-endian words w, OR base (whose bits SH..SH+BITS-1 are clear): a shift
// or a funnel shift that puts the code at bit SH, then one AND-OR.
template <int BITS, int C, int SH, int N>
__device__ __forceinline__ uint32_t code_addr(const uint32_t (&w)[N], uint32_t base) {
    constexpr int S = BITS * C - SH;
    static_assert(S + SH + BITS <= 32 * N, "code inside the words");
    uint32_t win;
    if constexpr (S < 0) win = w[0] << SH;
    else if constexpr (S % 32 + SH + BITS <= 32) win = w[S / 32] >> (S % 32);
    else win = __builtin_amdgcn_alignbit(w[S / 32 + 1], w[S / 32], S % 32);
    uint32_t r;
    // One v_and_or_b32 (left to itself the compiler splits it into an AND and an ADD).
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(win), "s"(((1u << BITS) - 1u) << SH), "v"(base));
    return r;
}
template <int C, int SH, int N>
__device__ __forceinline__ uint32_t code12_addr(const uint32_t (&w)[N], uint32_t base) {
    return code_addr<12, C, SH>(w, base);
}

// 1.5-bit: an 8-dim centroid is two 4-dim halves, so the same products run on
// 32 "virtual" sub-vectors j' = 2j + e of 4 dims (e = half).  A score lookup
// reads the whole 16-byte entry and feeds two products; a value lookup reads
// one 8-byte half (e = lane % 2 with the lane mapping above).  Books are single
// copies (2 x 64 KB).  Key codes are 24 bytes per token; value codes come in
// 48-byte streams, one per lane pair, 16 pairs (sub-vectors j, j + 8) in step
// order.
// 1.25-bit (2^10 x 8): the 1.5-bit products with 10-bit codes (keys 20 bytes
// per token, value streams of 40 bytes).  A 16 KB book leaves room for four
// copies in each 64 KB book region, copy c of entry e at 64 e + 16 c: score
// lookups take copy lane % 4 (the 16 lanes of a 16-byte read pass spread over
// four copies), value lookups copy (lane / 2) % 4 (a lane pair reads the two
// halves of one copy), which about halves the bank conflicts of random
// lookups into a single copy.
// 4-bit (2^8 x 2): the 2-bit products with each 4-dim operand made of the two
// 2-dim entries of sub-vectors 2w and 2w + 1.  A 1 KB book fills its 64 KB
// region as 64 copies, copy c of entry e at 256 e + 4 c, and lane l reads copy
// l (the 64 lanes of a 4-byte read hit 64 distinct banks).  Key codes are 64
// bytes per token; a value lookup's two entries are written as the lane's
// 8-byte row into a per-wave area and read back through the transposing read.
template <int FMT, int G, int NW, bool PAGED, bool APPEND = false>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeArgs a) {
    constexpr int HB = (G + 3) / 4;
    constexpr int PT_BYTES = NW * HB * 512;
    // 4-bit: 1 KB per wave where the value lookups are assembled into 4-dim
    // rows for the transposing read (16 bytes per lane: its rows for both
    // dims halves).
    constexpr int SV_BYTES = FMT == 4 ? NW * 1024 : 0;
    constexpr int MERGE_BYTES = NW * G * (kHeadDim + 2) * 4;
    // Fused append: both books widened to fp64 for its exact search (16 KB).
    constexpr int WIDE_BYTES = APPEND ? 2 * 256 * 4 * 8 : 0;
    constexpr int MAIN_BYTES = 2 * kBookBytes + PT_BYTES + SV_BYTES + WIDE_BYTES;
    constexpr int SMEM = MAIN_BYTES > MERGE_BYTES ? MAIN_BYTES : MERGE_BYTES;
    constexpr int W = FMT == 0 ? 32 : (FMT == 1 ? 24 : (FMT == 2 ? 48 : (FMT == 3 ? 20 : 64)));
    static_assert(FMT != 1 || 4096 * 16 == kBookBytes, "a 1.5-bit book fills one book region");
    static_assert(FMT != 3 || 1024 * 16 * 4 == kBookBytes, "four copies of a 1.25-bit book fill one region");
    static_assert(FMT != 2 || 4096 * 8 <= kBookBytes, "a 3-bit book fits one book region");
    static_assert(FMT != 4 || 256 * 64 * 4 == kBookBytes, "64 copies of a 4-bit book fill one region");
    __shared__ __align__(16) unsigned char smem[SMEM];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    // The wave index in a scalar register: the tile loop below is then
    // uniform control flow (the compiler cannot see that threadIdx.x / 64 is
    // the same in every lane of a wave).
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t_begin = s * a.chunk;
    const int t_end = min(seq_len_of(a, b), t_begin + a.chunk);

    // 2-bit and 1.25-bit: codebook entries are fetched into registers here and
    // written to LDS after the first tiles' code loads have been issued (loads
    // complete in order, so waiting for book loads issued after the code loads
    // would also wait for the codes, and the first tiles' latency would not
    // overlap the staging).  The 2-bit books come through the scalar path: wave
    // w reads entries [16 w, 16 w + 16) of each book (128 bytes, four 64-byte
    // scalar loads in all) into SGPRs, so they are not queued in the vector
    // memory pipeline behind the other waves' first code requests (batch-1
    // decode over 32k tokens 11.3 -> 9.8 us).  The 12-bit formats stage their
    // books directly: held in registers across the code loads, their 128 bytes
    // per lane spill.
    static_assert((FMT != 0 && FMT != 4) || NW == 16, "2-bit, 4-bit: 16 waves stage 16 entries each");
    static_assert(FMT != 3 || NW * 64 == 1024, "1.25-bit: one thread per book entry");
    constexpr int ND = FMT == 0 ? 32 : (FMT == 4 ? 16 : 1);
    uint32_t kd[ND], vd[ND];                                // 2-bit, 4-bit: the wave's 16 entries (SGPRs)
    uint4 kq3, vq3;                                         // 1.25-bit: entry threadIdx.x of each book
    if constexpr (FMT == 3) {
        kq3 = ((const uint4*)(a.k_book + (int64_t)h * 1024 * 8))[threadIdx.x];
        vq3 = ((const uint4*)(a.v_book + (int64_t)h * 1024 * 8))[threadIdx.x];
    } else if constexpr (FMT == 0) {
        typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
        const const_u32_ptr kbs = (const_u32_ptr)(a.k_book + (int64_t)h * 256 * 4) + wave * 32;
        const const_u32_ptr vbs = (const_u32_ptr)(a.v_book + (int64_t)h * 256 * 4) + wave * 32;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            kd[i] = kbs[i];
            vd[i] = vbs[i];
        }
    } else if constexpr (FMT == 4) {
        // 4-bit: wave w reads entries [16 w, 16 w + 16) of each book (one
        // 4-byte entry per dword) through the scalar path, as the 2-bit books.
        typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
        const const_u32_ptr kbs = (const_u32_ptr)(a.k_book + (int64_t)h * 256 * 2) + wave * 16;
        const const_u32_ptr vbs = (const_u32_ptr)(a.v_book + (int64_t)h * 256 * 2) + wave * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            kd[i] = kbs[i];
            vd[i] = vbs[i];
        }
    } else if constexpr (FMT == 2) {
        // 3-bit: single copies, 8-byte entries (4 dims).
        const uint2* kb = (const uint2*)(a.k_book + (int64_t)h * 4096 * 4);
        const uint2* vb = (const uint2*)(a.v_book + (int64_t)h * 4096 * 4);
        for (int i = threadIdx.x; i < 4096; i += NW * 64) {
            ((uint2*)smem)[i] = kb[i];
            ((uint2*)(smem + kBookBytes))[i] = vb[i];
        }
    } else {
        const uint4* kb = (const uint4*)(a.k_book + (int64_t)h * 4096 * 8);
        const uint4* vb = (const uint4*)(a.v_book + (int64_t)h * 4096 * 8);
        for (int i = threadIdx.x; i < 4096; i += NW * 64) {
            ((uint4*)smem)[i] = kb[i];
            ((uint4*)(smem + kBookBytes))[i] = vb[i];
        }
    }
    auto write_books = [&]() {
        if constexpr (FMT == 0) {
            // Slot 32 e + c holds copy c of entry e (256 bytes per entry): wave w
            // writes entries 16 w + 2 k (lanes 0..31, copy = lane) and 16 w + 2 k + 1
            // (lanes 32..63, copy = lane - 32).
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bool lo = lane < 32;
                const int slot = (16 * wave + 2 * k) * 32 + lane;
                ((uint2*)smem)[slot] = make_uint2(lo ? kd[4 * k] : kd[4 * k + 2], lo ? kd[4 * k + 1] : kd[4 * k + 3]);
                ((uint2*)(smem + kBookBytes))[slot] =
                    make_uint2(lo ? vd[4 * k] : vd[4 * k + 2], lo ? vd[4 * k + 1] : vd[4 * k + 3]);
            }
        } else if constexpr (FMT == 3) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ((uint4*)smem)[threadIdx.x * 4 + c] = kq3;
                ((uint4*)(smem + kBookBytes))[threadIdx.x * 4 + c] = vq3;
            }
        } else if constexpr (FMT == 4) {
            // Slot 64 e + c holds copy c of entry e (4 bytes; 256 bytes per
            // entry): wave w writes its 16 entries, lane = copy.
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                ((uint32_t*)smem)[(16 * wave + k) * 64 + lane] = kd[k];
                ((uint32_t*)(smem + kBookBytes))[(16 * wave + k) * 64 + lane] = vd[k];
            }
        }
    };
    float m[G];
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = kNegInf;
    float lsum[HB];                                         // head 4hb + lane % 4
    float4_t o[HB][2];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        lsum[hb] = 0.0f;
        o[hb][0] = o[hb][1] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int64_t stream = (int64_t)b * a.hkv + h;
    // Codes of tile tl (64 tokens, one block) start at byte toff(tl) of the
    // stream, or, paged, of the pool at the block the table names (clamped to
    // the pool, so no table entry can make the kernel read outside it).
    const uint8_t* kbase = PAGED ? a.k_codes : a.k_codes + stream * (int64_t)a.cap * W;
    const uint8_t* vbase = PAGED ? a.v_codes : a.v_codes + stream * (int64_t)a.cap * W;
    // The table is read-only here and the tile index is wave-uniform, so a
    // constant-address-space view lets the compiler use scalar loads: a vector
    // load of an entry would be counted with the code loads, and waiting for
    // it would drain every code load in flight.
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const const_i32_ptr btab = PAGED ? (const_i32_ptr)(a.block_table + stream * (int64_t)(a.cap >> 6)) : nullptr;
    auto toff = [&](int tl) -> int64_t {
        if constexpr (!PAGED) {
            return (int64_t)tl * W;
        } else {
            int blk = btab[tl >> 6];
            blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
            return (int64_t)blk * (64 * W);
        }
    };
    // 2-bit: 32 copies, lane l reads copy l % 32; the value book starts at 64 KB.
    // 1.5-bit: value lookups read half e = lane % 2 of the entry.
    // 1.25-bit: score lookups copy lane % 4, value lookups copy (lane / 2) % 4, half lane % 2.
    // 4-bit: 64 copies, lane l reads copy l (4-byte entries).
    const uint32_t kofs = FMT == 0   ? (uint32_t)(lane & 31) * 8
                          : FMT == 3 ? (uint32_t)(lane & 3) * 16
                          : FMT == 4 ? (uint32_t)lane * 4
                                     : 0u;
    const uint32_t vofs = (FMT == 0 || FMT == 4) ? (kofs | (1u << 16))
                          : FMT == 3 ? (((uint32_t)(lane >> 1) & 3u) * 16 | ((uint32_t)(lane & 1) << 3) | (1u << 16))
                          : FMT == 1 ? (((uint32_t)(lane & 1) << 3) | (1u << 16))
                                     : (1u << 16);
    unsigned char* pt = smem + 2 * kBookBytes + wave * (HB * 512);
    const int row_w = lane * 8;
    const int row_r = ((lane & 0x30) | ((lane & 3) << 2) | ((lane >> 2) & 3)) * 8;
    constexpr int P_LOG2 = 15;
    constexpr uint32_t kOnes = 0x3c003c00u;

    // Each code register is reloaded with a later tile's codes right after
    // its last use (at least a whole phase of work hides the load); the
    // tile index is clamped to a valid tile so the loads stay in bounds.
    constexpr int kStride = NW * 64;
    const int first = t_begin + wave * 64;
    // 2-bit: 32 bytes per lane per tile for keys and values.  1.5-bit: 24
    // bytes (3 x 8) of keys, 48 bytes (3 x 16) of values from stream
    // 8 (lane / 16) + 2 ((lane / 4) % 4) + (lane / 2) % 2 of the block.
    const int vstream = 8 * (lane >> 4) + 2 * ((lane >> 2) & 3) + ((lane >> 1) & 1);
    const uint8_t* kl0 = kbase + lane * 32;
    const uint8_t* vl0 = vbase + lane * 32;
    const uint8_t* kl1 = kbase + lane * 24;
    const uint8_t* vl1 = vbase + vstream * 48;
    // 3-bit: 48 bytes per lane per tile for keys (the lane's token) and
    // values (chunk = lane of the block).
    const uint8_t* kl2 = kbase + lane * 48;
    const uint8_t* vl2 = vbase + lane * 48;
    // 1.25-bit: 20 bytes (5 dwords) of the lane's token, 40 bytes (5 x 8) of its
    // lane pair's value stream (the 1.5-bit stream index).
    const uint8_t* kl3 = kbase + lane * 20;
    const uint8_t* vl3 = vbase + vstream * 40;
    // 4-bit: 64 bytes per lane per tile for keys (the lane's token) and values
    // (chunk = lane of the block).
    const uint8_t* kl4 = kbase + lane * 64;
    const uint8_t* vl4 = vbase + lane * 64;
    uint4 ck0, ck1, cv0, cv1;                               // 2-bit
    uint2 dk[3];                                            // 1.5-bit
    uint4 dv[3];
    uint4 ek[3], ev[3];                                     // 3-bit
    uint32_t fk[5];                                         // 1.25-bit
    uint2 fv[5];
    uint4 gk[4], gv[4];                                     // 4-bit
    auto load_k = [&](int tl) {
        if constexpr (FMT == 0) {
            const int64_t o = toff(tl);
            ck0 = *(const uint4*)(kl0 + o);
            ck1 = *(const uint4*)(kl0 + o + 16);
        } else if constexpr (FMT == 2) {
#pragma unroll
            for (int i = 0; i < 3; ++i) ek[i] = *(const uint4*)(kl2 + toff(tl) + 16 * i);
        } else if constexpr (FMT == 3) {
#pragma unroll
            for (int i = 0; i < 5; ++i) fk[i] = *(const uint32_t*)(kl3 + toff(tl) + 4 * i);
        } else if constexpr (FMT == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gk[i] = *(const uint4*)(kl4 + toff(tl) + 16 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 3; ++i) dk[i] = *(const uint2*)(kl1 + toff(tl) + 8 * i);
        }
    };
    auto load_v = [&](int tl) {
        if constexpr (FMT == 0) {
            const int64_t o = toff(tl);
            cv0 = *(const uint4*)(vl0 + o);
            cv1 = *(const uint4*)(vl0 + o + 16);
        } else if constexpr (FMT == 2) {
#pragma unroll
            for (int i = 0; i < 3; ++i) ev[i] = *(const uint4*)(vl2 + toff(tl) + 16 * i);
        } else if constexpr (FMT == 3) {
#pragma unroll
            for (int i = 0; i < 5; ++i) fv[i] = *(const uint2*)(vl3 + toff(tl) + 8 * i);
        } else if constexpr (FMT == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[i] = *(const uint4*)(vl4 + toff(tl) + 16 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 3; ++i) dv[i] = *(const uint4*)(vl1 + toff(tl) + 16 * i);
        }
    };
    // 2-bit: a second code set, so each tile's codes arrive two tiles ahead
    // (which matters when a wave has few tiles: six per wave at batch 1).
    uint4 bk0, bk1, bv0, bv1;
    // The first tile's codes, issued on every path: a wave without tiles
    // reads tile 0, which every stream has (capacity >= 64 tokens; paged,
    // table entries are clamped).  With a path that skips them, the waits the
    // compiler places for the query loads above would also cover these, and
    // the first tile's codes would have to arrive before the loop starts.
    // The loads go out in the loop's own order (keys, values; set A, then set
    // B in load_second), so the waits inside the loop are the same on the
    // first pass.
    auto load_first = [&]() {
        const int f = first < t_end ? first : 0;
        load_k(f);
        __builtin_amdgcn_sched_barrier(0);
        load_v(f);
    };
    // 2-bit: the second tile's codes (set B), issued after the prologue's
    // barrier.  With both tiles requested at kernel start (32 MB at batch 1)
    // the books, the query and the fused append's own loads queued behind
    // them; half as much ahead of the prologue made the batch-1 196k decode
    // 27.4 -> 26.5 us and its step 33.8 -> 32.1 us (interleaved A/B, one box;
    // batch 32 unchanged).
    auto load_second = [&]() {
        if constexpr (FMT == 0) {
            const int f = first < t_end ? first : 0;
            const int second = first + kStride < t_end ? first + kStride : f;
            const int64_t o = toff(second);
            __builtin_amdgcn_sched_barrier(0);
            bk0 = *(const uint4*)(kl0 + o);
            bk1 = *(const uint4*)(kl0 + o + 16);
            __builtin_amdgcn_sched_barrier(0);
            bv0 = *(const uint4*)(vl0 + o);
            bv1 = *(const uint4*)(vl0 + o + 16);
        }
    };
    bool loaded = false;
    // Query operands: lane 4c + i holds head 4hb + i's dims of (virtual)
    // sub-vector 16r + c, times sm_scale * log2(e), rounded to fp16.
    float4 qv[HB][2];
    auto fetch_q = [&](const float* qp) {
        const int c = lane >> 2, i = lane & 3;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int g = 4 * hb + i;
                qv[hb][r] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (g < G) qv[hb][r] = *(const float4*)(qp + g * kHeadDim + 4 * (16 * r + c));
            }
    };
    if constexpr (!APPEND) {
        // 2-bit: the query, then the first tiles' codes, then the books into
        // LDS; the waits for the books and the query leave the codes in flight.
        fetch_q(a.q_prime + ((int64_t)b * a.hq + h * G) * kHeadDim);
        if constexpr (FMT == 0 || FMT == 3 || FMT == 4) {
            __builtin_amdgcn_sched_barrier(0);
            load_first();
            loaded = true;
            __builtin_amdgcn_sched_barrier(0);
            write_books();
        }
    } else {
        // One-split decode step: q' and the new token's codes come first.
        static_assert(FMT == 0, "the fused append codes 2-bit tokens");
        static_assert(2 * kHeadDim * 8 + G * kHeadDim * 4 <= PT_BYTES, "rows and q' fit the probability tiles");
        double* xr = (double*)(smem + 2 * kBookBytes);
        float* qr = (float*)(smem + 2 * kBookBytes + 2 * kHeadDim * 8);
        // The append's own loads, then the wave's first tile, then the books
        // into LDS: the append's waits leave the code loads in flight.  If the
        // first tile holds the new token its codes are requested again after
        // the append (the first loads read the old bytes); the second tile is
        // requested after the append in any case (load_second).
        const AppendFetch af = fused_append_fetch<G, NW>(a, b, h);
        bool stale = false;
        if (af.app && first < t_end) {
            const int64_t nb = toff((int)(af.t & ~(int64_t)63));
            stale = toff(first) == nb;
        }
        __builtin_amdgcn_sched_barrier(0);
        load_first();
        loaded = !stale;
        __builtin_amdgcn_sched_barrier(0);
        write_books();
        fused_append_2bit<G, NW>(a, b, h, af, xr, qr, smem,
                                 (double*)(smem + 2 * kBookBytes + PT_BYTES + SV_BYTES));
        fetch_q(qr);
    }
    // The query operand in fp16 range: head g's q' * qscale is scaled by
    // 2^-k_g, k_g >= 0 the smallest that brings every element below 2^15, and
    // its scores are taken back by 2^k_g in the exponents and when m leaves
    // the kernel (powers of two: exact).  k_g = 0 for queries of attention's
    // usual size, and then every result is what it is without this step.
    // Lanes with equal lane % 4 hold one head's elements.
    half4_t qa[HB][2];
    float qsc[G];                                           // 2^k_g, wave-uniform
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        float mx = 0.0f;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float4 q = qv[hb][r];
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(q.x * a.qscale), fabsf(q.y * a.qscale)),
                                 fmaxf(fabsf(q.z * a.qscale), fabsf(q.w * a.qscale))));
        }
        mx = fmaxf(mx, xor_lane(mx, 4));
        mx = fmaxf(mx, xor_lane(mx, 8));
        mx = fmaxf(mx, xor_lane(mx, 16));
        mx = fmaxf(mx, xor_lane(mx, 32));
        int e = 0;
        if (__builtin_isfinite(mx)) (void)frexpf(mx, &e);  // mx < 2^e; a non-finite query keeps k = 0
        const int k = e > 15 ? e - 15 : 0;
        const float inv = ldexpf(1.0f, -k);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * hb + i < G) qsc[4 * hb + i] = readlane(ldexpf(1.0f, k), i);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float4 q = qv[hb][r];
            qa[hb][r] = half4_t{(_Float16)(q.x * a.qscale * inv), (_Float16)(q.y * a.qscale * inv),
                                (_Float16)(q.z * a.qscale * inv), (_Float16)(q.w * a.qscale * inv)};
        }
    }
    __syncthreads();
    if (!loaded) load_first();
    load_second();

    // One tile; the 2-bit code registers are parameters so that two sets can
    // alternate (codes loaded two tiles ahead).
    auto step = [&](int tile, int nxt, uint4& ck0, uint4& ck1, uint4& cv0, uint4& cv1) {
        const int t = tile + lane;
        float4_t sacc[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sacc[hb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (FMT == 0) {
            // Scores: 32 sub-vectors, 16 per code half.
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint4 ck = half == 0 ? ck0 : ck1;
                const uint32_t kw[4] = {ck.x, ck.y, ck.z, ck.w};
                static_for<0, 16>([&](auto jc) {
                    constexpr int jj = decltype(jc)::value;     // sub-vector 16 * half + jj
                    const uint32_t addr = __builtin_amdgcn_perm(kw[jj >> 2], kofs, lookup_sel<jj & 3>());
                    const half4_t kv = *(const half4_t*)(smem + addr);
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) sacc[hb] = mfma_bcast<jj>(qa[hb][half], kv, sacc[hb]);
                });
                __builtin_amdgcn_sched_barrier(0);
                if (half == 0) ck0 = *(const uint4*)(kl0 + toff(nxt));
                else ck1 = *(const uint4*)(kl0 + toff(nxt) + 16);
            }
        } else if constexpr (FMT == 4) {
            // Scores: 32 groups of 4 dims; group w is sub-vectors 2w and 2w + 1,
            // bytes 2w and 2w + 1 of the lane's 64 bytes: two 4-byte lookups
            // make the B operand of the 2-bit path's sub-vector w.
            const uint32_t kw[16] = {gk[0].x, gk[0].y, gk[0].z, gk[0].w, gk[1].x, gk[1].y, gk[1].z, gk[1].w,
                                     gk[2].x, gk[2].y, gk[2].z, gk[2].w, gk[3].x, gk[3].y, gk[3].z, gk[3].w};
            static_for<0, 32>([&](auto wc) {
                constexpr int w = decltype(wc)::value;
                const uint32_t a0 = __builtin_amdgcn_perm(kw[w >> 1], kofs, lookup_sel<2 * (w & 1)>());
                const uint32_t a1 = __builtin_amdgcn_perm(kw[w >> 1], kofs, lookup_sel<2 * (w & 1) + 1>());
                const half4_t kv =
                    __builtin_bit_cast(half4_t, make_uint2(*(const uint32_t*)(smem + a0), *(const uint32_t*)(smem + a1)));
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) sacc[hb] = mfma_bcast<w & 15>(qa[hb][w >> 4], kv, sacc[hb]);
            });
            __builtin_amdgcn_sched_barrier(0);
            load_k(nxt);
        } else if constexpr (FMT == 2) {
            // Scores: 32 sub-vectors; the 12-bit code of sub-vector j sits at
            // bit 12 j of the lane's 48 bytes.
            const uint32_t kw[12] = {ek[0].x, ek[0].y, ek[0].z, ek[0].w, ek[1].x, ek[1].y,
                                     ek[1].z, ek[1].w, ek[2].x, ek[2].y, ek[2].z, ek[2].w};
            static_for<0, 32>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const uint32_t addr = code12_addr<j, 3>(kw, 0u);
                const half4_t kv = *(const half4_t*)(smem + addr);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) sacc[hb] = mfma_bcast<j & 15>(qa[hb][j >> 4], kv, sacc[hb]);
            });
            __builtin_amdgcn_sched_barrier(0);
            load_k(nxt);
        } else {
            // Scores: 16 sub-vectors in 8 pairs; each 16-byte entry feeds the
            // products of virtual sub-vectors 2j and 2j + 1.  12-bit codes of
            // 24 bytes (1.5-bit), or 10-bit codes of 20 bytes at 64-byte entry
            // strides (1.25-bit, four copies).
            constexpr int CB = FMT == 3 ? 10 : 12, CSH = FMT == 3 ? 6 : 4, NKW = FMT == 3 ? 5 : 6;
            uint32_t kw[NKW];
            if constexpr (FMT == 3) {
#pragma unroll
                for (int i = 0; i < 5; ++i) kw[i] = fk[i];
            } else {
                kw[0] = dk[0].x; kw[1] = dk[0].y; kw[2] = dk[1].x; kw[3] = dk[1].y; kw[4] = dk[2].x; kw[5] = dk[2].y;
            }
            static_for<0, 8>([&](auto mc) {
                constexpr int mp = decltype(mc)::value;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const uint32_t addr = u == 0 ? code_addr<CB, 2 * mp, CSH>(kw, kofs)
                                                 : code_addr<CB, 2 * mp + 1, CSH>(kw, kofs);
                    const uint4 ent = *(const uint4*)(smem + addr);
                    const half4_t lo = __builtin_bit_cast(half4_t, make_uint2(ent.x, ent.y));
                    const half4_t hi = __builtin_bit_cast(half4_t, make_uint2(ent.z, ent.w));
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) {
                        // virtual sub-vectors 4 mp + 2u and 4 mp + 2u + 1, both in register pair mp / 4
                        if (u == 0) {
                            sacc[hb] = mfma_bcast<(4 * mp) & 15>(qa[hb][mp >> 2], lo, sacc[hb]);
                            sacc[hb] = mfma_bcast<(4 * mp + 1) & 15>(qa[hb][mp >> 2], hi, sacc[hb]);
                        } else {
                            sacc[hb] = mfma_bcast<(4 * mp + 2) & 15>(qa[hb][mp >> 2], lo, sacc[hb]);
                            sacc[hb] = mfma_bcast<(4 * mp + 3) & 15>(qa[hb][mp >> 2], hi, sacc[hb]);
                        }
                    }
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            load_k(nxt);
        }
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = t < t_end ? sacc[g >> 2][g & 3] : kNegInf;
        float p[G];
        softmax_tile_lazy_scaled<G, P_LOG2>(sc, m, qsc, p, [&](int g, float alpha) {
            o[g >> 2][0][g & 3] *= alpha;
            o[g >> 2][1][g & 3] *= alpha;
            if ((lane & 3) == (g & 3)) lsum[g >> 2] *= alpha;
        });
        // Probabilities to lane 4s + i = head i, tokens 4s..4s+3.
        half4_t pt_op[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            half4_t v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = 4 * hb + i < G ? (_Float16)p[4 * hb + i] : (_Float16)0.0f;
            *(half4_t*)(pt + hb * 512 + row_w) = v;
        }
        wave_lds_sync();
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            pt_op[hb] = lds_read_tr16((const lds_char*)(pt + hb * 512 + row_r));
            const uint2 pw = __builtin_bit_cast(uint2, pt_op[hb]);
            lsum[hb] = dot2(pw.x, kOnes, dot2(pw.y, kOnes, lsum[hb]));
        }
        if constexpr (FMT == 0) {
            // Values: step st takes byte 2 st + half of the lane's code chunk.
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                const uint4 cv = hv == 0 ? cv0 : cv1;
                const uint32_t vw[4] = {cv.x, cv.y, cv.z, cv.w};
                static_for<0, 8>([&](auto sc8) {
                    constexpr int st8 = decltype(sc8)::value;   // step 8 * hv + st8
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const uint32_t sel = hh == 0 ? lookup_sel<2 * (st8 & 1)>() : lookup_sel<2 * (st8 & 1) + 1>();
                        const uint32_t addr = __builtin_amdgcn_perm(vw[st8 >> 1], vofs, sel);
                        const half4_t vv = lds_read_tr16((const lds_char*)(smem + addr));
#pragma unroll
                        for (int hb = 0; hb < HB; ++hb) {
                            if (hv == 0) o[hb][hh] = mfma_bcast<st8>(pt_op[hb], vv, o[hb][hh]);
                            else o[hb][hh] = mfma_bcast<8 + st8>(pt_op[hb], vv, o[hb][hh]);
                        }
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
                if (hv == 0) cv0 = *(const uint4*)(vl0 + toff(nxt));
                else cv1 = *(const uint4*)(vl0 + toff(nxt) + 16);
            }
        } else if constexpr (FMT == 4) {
            // Values: lane 16r + 4k + q takes, at step st, dword st of its
            // chunk: the codes of token 4 st + k, sub-vectors 2w and 2w + 1 with
            // w = 16 hh + 4r + q, for dims half hh = 0 (bytes 0, 1) and hh = 1
            // (bytes 2, 3).  Its two 4-byte entries are written as the lane's
            // 8-byte row (dims 4w..4w+3 of the token) and read back through the
            // transposing read, which hands block 4r + q the same (token x dim)
            // operand the 2-bit path's direct lookup does.
            const uint32_t vw[16] = {gv[0].x, gv[0].y, gv[0].z, gv[0].w, gv[1].x, gv[1].y, gv[1].z, gv[1].w,
                                     gv[2].x, gv[2].y, gv[2].z, gv[2].w, gv[3].x, gv[3].y, gv[3].z, gv[3].w};
            // The lane's two rows (hh = 0, 1) are adjacent: one 16-byte write.
            unsigned char* rows = smem + 2 * kBookBytes + PT_BYTES + wave * 1024 + lane * 16;
            static_for<0, 16>([&](auto sc16) {
                constexpr int st = decltype(sc16)::value;
                uint32_t e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t sel = i == 0 ? lookup_sel<0>() : (i == 1 ? lookup_sel<1>() : (i == 2 ? lookup_sel<2>() : lookup_sel<3>()));
                    e[i] = *(const uint32_t*)(smem + __builtin_amdgcn_perm(vw[st], vofs, sel));
                }
                *(uint4*)rows = make_uint4(e[0], e[1], e[2], e[3]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const half4_t vv = lds_read_tr16((const lds_char*)(rows + hh * 8));
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) o[hb][hh] = mfma_bcast<st>(pt_op[hb], vv, o[hb][hh]);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            load_v(nxt);
        } else if constexpr (FMT == 2) {
            // Values: step st takes the pair (sub-vector j, j + 16) of token
            // group st, bytes 3 st.. of the lane's chunk (j % 16 fixed by the lane).
            const uint32_t vw[12] = {ev[0].x, ev[0].y, ev[0].z, ev[0].w, ev[1].x, ev[1].y,
                                     ev[1].z, ev[1].w, ev[2].x, ev[2].y, ev[2].z, ev[2].w};
            static_for<0, 16>([&](auto sc16) {
                constexpr int st = decltype(sc16)::value;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t addr = hh == 0 ? code12_addr<2 * st, 3>(vw, vofs) : code12_addr<2 * st + 1, 3>(vw, vofs);
                    const half4_t vv = lds_read_tr16((const lds_char*)(smem + addr));
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) o[hb][hh] = mfma_bcast<st>(pt_op[hb], vv, o[hb][hh]);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            load_v(nxt);
        } else {
            // Values: step st takes pair st of the lane's stream (bits 24 st..,
            // 1.5-bit; bits 20 st.., 1.25-bit).
            constexpr int CB = FMT == 3 ? 10 : 12, CSH = FMT == 3 ? 6 : 4, NVW = FMT == 3 ? 10 : 12;
            uint32_t vw[NVW];
            if constexpr (FMT == 3) {
#pragma unroll
                for (int i = 0; i < 5; ++i) { vw[2 * i] = fv[i].x; vw[2 * i + 1] = fv[i].y; }
            } else {
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    vw[4 * i] = dv[i].x; vw[4 * i + 1] = dv[i].y; vw[4 * i + 2] = dv[i].z; vw[4 * i + 3] = dv[i].w;
                }
            }
            static_for<0, 16>([&](auto sc16) {
                constexpr int st = decltype(sc16)::value;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t addr = hh == 0 ? code_addr<CB, 2 * st, CSH>(vw, vofs)
                                                  : code_addr<CB, 2 * st + 1, CSH>(vw, vofs);
                    const half4_t vv = lds_read_tr16((const lds_char*)(smem + addr));
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) o[hb][hh] = mfma_bcast<st>(pt_op[hb], vv, o[hb][hh]);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            load_v(nxt);
        }
        wave_lds_sync();
    };
    if constexpr (FMT == 0) {
        // Whole pairs of tiles in the loop, an odd last tile after it: the
        // loop header is reached only after set B's loads, so the wait before
        // set A's first use lets all seven younger loads stay in flight (with
        // a skippable second step in the loop the compiler also waited for
        // set B's first load, i.e. codes requested half a tile earlier).
        const int ntiles = first < t_end ? (t_end - first + kStride - 1) / kStride : 0;
        // The waves of a work-group are kept in step: the instruction arbiter
        // favours the oldest wave of each SIMD, and left alone the four age
        // groups drift apart (at 192 tiles per wave the youngest finished
        // ~40% of the pass after the oldest, leaving fewer waves with loads
        // in flight).  A bare s_barrier (no memory fence, so no wait for the
        // code loads) every kSyncTiles tiles, up to the tile count of the last
        // wave, which has the fewest: every wave executes the same barriers.
        constexpr int kSyncTiles = 16;
        const int last_first = t_begin + (NW - 1) * 64;
        const int nmin = last_first < t_end ? (t_end - last_first + kStride - 1) / kStride : 0;
        int tile = first;
        for (int it = 0; it < (ntiles >> 1); ++it) {
            step(tile, tile + 2 * kStride < t_end ? tile + 2 * kStride : tile, ck0, ck1, cv0, cv1);
            const int t2 = tile + kStride;
            step(t2, t2 + 2 * kStride < t_end ? t2 + 2 * kStride : t2, bk0, bk1, bv0, bv1);
            tile += 2 * kStride;
            if ((2 * (it + 1)) % kSyncTiles == 0 && 2 * (it + 1) <= nmin) __builtin_amdgcn_s_barrier();
        }
        if (ntiles & 1) step(tile, tile, ck0, ck1, cv0, cv1);
    } else {
        for (int tile = first; tile < t_end; tile += kStride)
            step(tile, tile + kStride < t_end ? tile + kStride : tile, ck0, ck1, cv0, cv1);
    }

    float l[G];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        float x = lsum[hb];
        x += xor_lane(x, 4);
        x += xor_lane(x, 8);
        x += xor_lane(x, 16);
        x += xor_lane(x, 32);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * hb + i < G) l[4 * hb + i] = readlane(x, i);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] *= qsc[g];             // back to true score units
    __syncthreads();
    float* scratch = (float*)smem;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        scratch[(wave * G + g) * kHeadDim + lane] = o[g >> 2][0][g & 3];
        scratch[(wave * G + g) * kHeadDim + 64 + lane] = o[g >> 2][1][g & 3];
    }
    stash_ml<G, NW>(scratch, m, l);
    __syncthreads();
    float* stage = scratch + NW * G * (kHeadDim + 2);       // after the merge scratch
    static_assert(SMEM >= MERGE_BYTES + G * (kHeadDim + 2) * 4, "LDS holds the merge scratch and the stage");
    merge_waves<G, NW>(scratch, a, b, h, s, (float)P_LOG2, stage);
    if (a.out != nullptr && a.splits > 1) {
        combine_if_last<G, NW>(smem, stage, a, b, h);
    } else if (a.out != nullptr && a.v_smooth != nullptr) {
        // One split of the value-transform variant: the merged o (staged in LDS)
        // mapped back, one wave per query head.
        __syncthreads();
        if (wave < G)
            value_untransform_wave(stage + kHeadDim * wave, a.v_smooth + (int64_t)h * kHeadDim,
                                   a.out + ((int64_t)b * a.hq + h * G + wave) * kHeadDim, lane);
    }
}

// ------------------------------------------------------------------ gather path

template <int FMT, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_gather_kernel(DecodeArgs a) {
    using F = DFmt<FMT>;
    constexpr int E = F::E, DS = F::DS, J = F::J, W = F::W;
    constexpr int BOOK_BYTES = E * DS * 2;
    constexpr int MERGE_BYTES = NW * G * (kHeadDim + 2) * 4;
    constexpr int A_BYTES = BOOK_BYTES > MERGE_BYTES ? BOOK_BYTES : MERGE_BYTES;
    constexpr int HB = (G + 3) / 4;
    __shared__ __align__(16) unsigned char region_a[A_BYTES];      // K book, then merge scratch
    __shared__ __align__(16) uint16_t vbook[E * DS];
    __shared__ __align__(16) float qs[G * kHeadDim];
    __shared__ __align__(16) uint32_t pbuf[NW][16 * 8 * HB];       // fp16 A operands of the value product
    uint16_t* kbook = (uint16_t*)region_a;

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t_begin = s * a.chunk;
    const int t_end = min(seq_len_of(a, b), t_begin + a.chunk);

    {
        const uint4* kb = (const uint4*)(a.k_book + (int64_t)h * E * DS);
        const uint4* vb = (const uint4*)(a.v_book + (int64_t)h * E * DS);
        for (int i = threadIdx.x; i < E * DS / 8; i += NW * 64) {
            ((uint4*)kbook)[i] = kb[i];
            ((uint4*)vbook)[i] = vb[i];
        }
        const float* qp = a.q_prime + ((int64_t)b * a.hq + h * G) * kHeadDim;
        for (int i = threadIdx.x; i < G * kHeadDim; i += NW * 64) qs[i] = qp[i] * a.qscale;
        if (G % 4 != 0)                                      // padding heads stay zero
            for (int i = threadIdx.x; i < NW * 16 * 8 * HB; i += NW * 64) (&pbuf[0][0])[i] = 0u;
    }
    __syncthreads();

    float m[G], l[G];
    float4_t o[HB][2];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) o[hb][0] = o[hb][1] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int P_LOG2 = 15;                               // p and l carry 2^15
    const int64_t stream = (int64_t)b * a.hkv + h;
    const uint8_t* kbase = a.k_codes + stream * (int64_t)a.cap * W;
    const uint8_t* vbase = a.v_codes + stream * (int64_t)a.cap * W;
    uint32_t* pw = pbuf[wave];
    const lds_char* vt = (const lds_char*)vbook;
    const uint32_t eofs = FMT == 0 ? 0u : (uint32_t)(lane & 1) * 8;   // 1.5-bit: half of the entry
    const int vstream = 8 * (lane >> 4) + 2 * ((lane >> 2) & 3) + ((lane >> 1) & 1);

    for (int tile = t_begin + wave * 64; tile < t_end; tile += NW * 64) {
        const int t = tile + lane;
        // Key codes of this lane's token; value codes of its chunk or stream.
        uint32_t kw[W / 4], vw[FMT == 0 ? 8 : 12];
        if constexpr (FMT == 0) {
            const uint4* kc = (const uint4*)(kbase + (int64_t)t * 32);
            const uint4 k0 = kc[0], k1 = kc[1];
            kw[0] = k0.x; kw[1] = k0.y; kw[2] = k0.z; kw[3] = k0.w;
            kw[4] = k1.x; kw[5] = k1.y; kw[6] = k1.z; kw[7] = k1.w;
            const uint4* vc = (const uint4*)(vbase + (int64_t)tile * 32 + lane * 32);
            const uint4 v0 = vc[0], v1 = vc[1];
            vw[0] = v0.x; vw[1] = v0.y; vw[2] = v0.z; vw[3] = v0.w;
            vw[4] = v1.x; vw[5] = v1.y; vw[6] = v1.z; vw[7] = v1.w;
        } else {
            const uint2* kc = (const uint2*)(kbase + (int64_t)t * 24);
            const uint2 k0 = kc[0], k1 = kc[1], k2 = kc[2];
            kw[0] = k0.x; kw[1] = k0.y; kw[2] = k1.x; kw[3] = k1.y; kw[4] = k2.x; kw[5] = k2.y;
            const uint4* vc = (const uint4*)(vbase + (int64_t)tile * 24 + vstream * 48);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const uint4 v = vc[i];
                vw[4 * i] = v.x; vw[4 * i + 1] = v.y; vw[4 * i + 2] = v.z; vw[4 * i + 3] = v.w;
            }
        }
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = 0.0f;
        // Scores: gather the token's centroids, fp32 dot products with q'.
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
        softmax_tile_lazy<G, P_LOG2>(sc, m, p, [&](int g, float alpha) {
            l[g] *= alpha;
            o[g >> 2][0][g & 3] *= alpha;
            o[g >> 2][1][g & 3] *= alpha;
        });
        store_probs<G, HB>(pw, p, l, lane);
        wave_lds_sync();
        // Values on the matrix cores (same lane mapping as the matrix-core kernel).
        static_for<0, 16>([&](auto sc16) {
            constexpr int st = decltype(sc16)::value;
            half4_t pa[HB];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
                pa[hb] = *(const half4_t*)((const char*)pw + st * 32 * HB + (4 * hb + (lane & 3)) * 8);
            uint32_t x = 0;
            if constexpr (FMT == 1) x = bytes3_at<3 * st>(vw);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint32_t addr;
                if constexpr (FMT == 0) addr = byte_at(vw, 2 * st + hh) * 8;
                else addr = (hh == 0 ? ((x << 4) & 0xfff0u) : ((x >> 8) & 0xfff0u)) | eofs;
                const half4_t vb = lds_read_tr16(vt + addr);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) o[hb][hh] = mfma_4x4x4(pa[hb], vb, o[hb][hh]);
            }
        });
        wave_lds_sync();
    }

#pragma unroll
    for (int g = 0; g < G; ++g) l[g] = 0.5f * wave_sum(l[g]);
    __syncthreads();
    float* scratch = (float*)region_a;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        scratch[(wave * G + g) * kHeadDim + lane] = o[g >> 2][0][g & 3];
        scratch[(wave * G + g) * kHeadDim + 64 + lane] = o[g >> 2][1][g & 3];
    }
    stash_ml<G, NW>(scratch, m, l);
    __syncthreads();
    merge_waves<G, NW>(scratch, a, b, h, s, (float)P_LOG2);
}

// ----------------------------------------------------------------------- combine

// One block per (b, q-head), thread d = output dim (combine_row).
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
    __shared__ float red[2], wts[128];
    combine_row(a.part_o, a.part_ml, a.out, a.splits, blockIdx.x, threadIdx.x, true, red, wts);
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
    // The matrix-core kernel unless a measurement override asks for the
    // score-table (2-bit, G <= 4) or gather kernel.
    if (a.out != nullptr && (a.path == 1 || a.path == 2)) return hipErrorInvalidValue;   // fused combine: matrix-core kernel
    if (a.fmt == 0 && a.path == 1) {
        if (a.block_table) return hipErrorInvalidValue;
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
    if (a.app.k_new != nullptr) {
        // Fused append, 2-bit: one split writes the output itself, several write
        // the splits' partials for the combine kernel.
        if (a.fmt != 0 || a.path != 3 || a.seq_lens || (a.splits == 1) != (a.out != nullptr)) return hipErrorInvalidValue;
        constexpr int NW = 16;
        const bool paged = a.block_table != nullptr;
#define VQKV_G(GV) case GV:                                                                                          \
            if (paged) hipLaunchKernelGGL((decode_mfma_kernel<0, GV, NW, true, true>), grid, dim3(NW * 64), 0, stream, a); \
            else hipLaunchKernelGGL((decode_mfma_kernel<0, GV, NW, false, true>), grid, dim3(NW * 64), 0, stream, a);      \
            break;
        switch (G) {
            VQKV_G(1) VQKV_G(2) VQKV_G(3) VQKV_G(4) VQKV_G(5) VQKV_G(6) VQKV_G(7) VQKV_G(8)
            default: return hipErrorInvalidValue;
        }
#undef VQKV_G
        return hipGetLastError();
    }
    if (a.path != 2) {
        constexpr int NW = 16;
        const bool paged = a.block_table != nullptr;
#define VQKV_G(F, GV) case GV:                                                                                     \
            if (paged) hipLaunchKernelGGL((decode_mfma_kernel<F, GV, NW, true>), grid, dim3(NW * 64), 0, stream, a); \
            else hipLaunchKernelGGL((decode_mfma_kernel<F, GV, NW, false>), grid, dim3(NW * 64), 0, stream, a);      \
            break;
        if (a.fmt == 0) {
            switch (G) {
                VQKV_G(0, 1) VQKV_G(0, 2) VQKV_G(0, 3) VQKV_G(0, 4) VQKV_G(0, 5) VQKV_G(0, 6) VQKV_G(0, 7) VQKV_G(0, 8)
                default: return hipErrorInvalidValue;
            }
        } else if (a.fmt == 1) {
            switch (G) {
                VQKV_G(1, 1) VQKV_G(1, 2) VQKV_G(1, 3) VQKV_G(1, 4) VQKV_G(1, 5) VQKV_G(1, 6) VQKV_G(1, 7) VQKV_G(1, 8)
                default: return hipErrorInvalidValue;
            }
        } else if (a.fmt == 2) {
            switch (G) {
                VQKV_G(2, 1) VQKV_G(2, 2) VQKV_G(2, 3) VQKV_G(2, 4) VQKV_G(2, 5) VQKV_G(2, 6) VQKV_G(2, 7) VQKV_G(2, 8)
                default: return hipErrorInvalidValue;
            }
        } else if (a.fmt == 3) {
            switch (G) {
                VQKV_G(3, 1) VQKV_G(3, 2) VQKV_G(3, 3) VQKV_G(3, 4) VQKV_G(3, 5) VQKV_G(3, 6) VQKV_G(3, 7) VQKV_G(3, 8)
                default: return hipErrorInvalidValue;
            }
        } else {
            switch (G) {
                VQKV_G(4, 1) VQKV_G(4, 2) VQKV_G(4, 3) VQKV_G(4, 4) VQKV_G(4, 5) VQKV_G(4, 6) VQKV_G(4, 7) VQKV_G(4, 8)
                default: return hipErrorInvalidValue;
            }
        }
#undef VQKV_G
        return hipGetLastError();
    }
    if (a.block_table || a.fmt >= 2) return hipErrorInvalidValue;   // matrix-core kernel only
    if (a.fmt == 0) return launch_gather<0, 8>(a, grid, stream);
    return launch_gather<1, 8>(a, grid, stream);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(combine_kernel, dim3(a.batch * a.hq), dim3(128), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vqkv
