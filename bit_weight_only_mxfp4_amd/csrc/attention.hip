// attention.hip -- single-token grouped-query attention over a bf16 KV cache
// (kerbin.cskartikey.dev/@satvikhardat, "Dev Log #3 -- SmolLM3-3B Results":
// each query head h reads kv head h / (hq / hkv); a score is the key . query
// dot product times the scale; the output is the softmax-weighted sum of the
// values over the cached positions).
//
// Split over positions (flash-decoding style), two kernels:
//  1. k_attn_partial, one wave per (64-position chunk, kv head): the G query
//     heads of the kv head against the chunk's keys and values on the bf16
//     matrix cores (scores K Q^T, then P V), scores in base-2 units
//     (s * scale * log2(e), so each exponential is one v_exp_f32), positions
//     past T read zeros and score -inf.  The chunk's (max, sum p, sum p V)
//     per head go to the caller's workspace.
//  2. k_attn_combine, one wave per (query head, 16 output columns): rescales
//     the chunks to the global maximum and sums them in chunk order (fixed
//     order: the result is the same on every run).
// A context of at most 256 / D chunks runs as one launch instead: one
// workgroup per kv head, one wave per chunk, merged through LDS.  Chunks are
// 64 positions, 32 for the split at contexts up to 2048.
#include <atomic>
#include <mutex>

#include "device.h"
#include "tt_internal.h"

namespace tt {

#ifndef TT_ATTN_CHUNK
#define TT_ATTN_CHUNK 64
#endif
constexpr int kAttnChunk = TT_ATTN_CHUNK;  // positions per chunk (a multiple of 32)
constexpr int kAttnOob = 0x7FFFFF00;
// A context of at most 256 / D chunks (64 KiB of keys and values per kv
// head) takes one workgroup of that many waves per kv head and no combine;
// longer contexts split over one-wave workgroups.
template <int D> constexpr int attn_single_waves() { return 256 / D; }

struct AttnArgs {
    const uint16_t *q, *k, *v;  // q [hq][d]; k, v [hkv][tcap][d]
    int32_t hq, hkv, tcap, T, nchunks;
    float scale2;               // scale * log2(e): scores in base-2 units
    float *part;                // [hkv][nchunks][G][D]
    float *ml;                  // [hkv][nchunks][G][2]: chunk max, chunk sum
    void *out;                  // [hq][d]
    int32_t out_bf16;
};

// The argument struct with the leading kernel parameters written in: the
// fields both kernels read before their first cache or workspace loads come
// preloaded in scalar registers; the output pointer comes with the struct.
__device__ __forceinline__ AttnArgs attn_hot_args(AttnArgs a, const uint16_t *q,
                                                  const uint16_t *k, const uint16_t *v,
                                                  float *part, float *ml, int32_t tcap, int32_t T,
                                                  int32_t nchunks, float scale2) {
    a.q = q;
    a.k = k;
    a.v = v;
    a.part = part;
    a.ml = ml;
    a.tcap = tcap;
    a.T = T;
    a.nchunks = nchunks;
    a.scale2 = scale2;
    return a;
}

__device__ __forceinline__ uint4 attn_load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

// Chunk pass, one wave per (16 NB positions, kv head).  Scores: S = K Q^T
// on v_mfma_f32_16x16x32_bf16 per block of 16 positions, A = the key rows
// (lane l: position l % 16, d = 32 kk + 8 (l / 16) .. +7: one 16-byte LDS
// read),
// B = the G query heads of the kv head as columns (heads past G are zero
// columns); lane (head c, group q) gets positions 4q .. 4q+3 of the block.
// The wave's maximum per head and p = exp2(s - max) stay in that layout,
// which is the A layout of the next product: P V on the same instruction
// with 32 positions per step (block 2m in elements 0..3, block 2m+1 in
// 4..7), P split into bf16 hi + lo parts (p - hi is exact in fp32 and its
// bf16 rounding leaves a 2^-18 relative residue) and V as B.  K and V go to
// LDS by buffer->LDS DMA (contiguous 1 KiB per instruction) in their
// row-major layout with the 16-byte chunks of row r xor-swizzled; K comes
// back by plain 16-byte reads, V as B operands through ds_read_b64_tr_b16:
// within each group of 16 lanes, source lane 4j + a addresses row j,
// columns 4a .. 4a+3 of a 4 x 16 tile, and lane i receives column i, rows
// 0..3.  No barrier across waves and no cross-lane reduction of P V.
template <int D>
__device__ __forceinline__ int attn_swz(int r) {
    return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

// W = 1: one wave per (chunk, kv head), partials to the workspace for the
// combine.  W > 1 (contexts of at most W chunks): one workgroup of W waves per
// kv head, wave w taking chunk w; waves 1 .. W-1 hand (max, sum, P V) to wave
// 0 through LDS, which rescales each part to the common maximum, adds them in
// wave order and writes the normalised output -- one launch for the call.
template <int D, int G, int NB, int W>
__global__ __launch_bounds__(64 * W) void k_attn_partial(const uint16_t *q, const uint16_t *k,
                                                        const uint16_t *v, float *part, float *ml,
                                                        int32_t tcap, int32_t T, int32_t nchunks,
                                                        float scale2, AttnArgs cold) {
    const AttnArgs a = attn_hot_args(cold, q, k, v, part, ml, tcap, T, nchunks, scale2);
    static_assert(NB % 2 == 0, "blocks of 16 positions come in pairs");
    constexpr int KK = D / 32;           // score steps over d
    constexpr int CPR = D / 8;           // 16-byte chunks per V row
    constexpr int NV = 16 * NB * CPR / 64;  // V DMA instructions
    constexpr int NT = D / 16;           // output column tiles
    __shared__ __attribute__((aligned(16))) uint16_t s_kw[W][16 * NB * D];
    __shared__ __attribute__((aligned(16))) uint16_t s_vw[W][16 * NB * D];
    __shared__ f32x4_t s_o[W > 1 ? W - 1 : 1][W > 1 ? NT : 1][64];
    __shared__ float s_ml[W][2][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint16_t *s_k = s_kw[wave], *s_v = s_vw[wave];
    const int c = blockIdx.x, g = blockIdx.y;
    const int t0 = (c * W + wave) * 16 * NB;
    const int col = lane & 15, grp = lane >> 4;

    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.q + (int64_t)g * G * D), 0, G * D * 2, 0x00020000);
    const int64_t head_off = (int64_t)g * a.tcap * D;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.k + head_off), 0, a.T * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.v + head_off), 0, a.T * D * 2, 0x00020000);

    // 1. query columns from memory; the chunk's key rows, then its value
    //    rows, into LDS by DMA (rows past T read zeros)
    uint4 qb[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qb[kk] = attn_load16(qr, col < G ? (col * D + 32 * kk + 8 * grp) * 2 : kAttnOob);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int L = u * 64 + lane, r = L / CPR, x = (L % CPR) ^ attn_swz<D>(r);
        const int t = t0 + r;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void *)(s_k + u * 512), 16,
            t < a.T ? (t * D + 8 * x) * 2 : kAttnOob, 0, 0, kStreamPolicy);
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int L = u * 64 + lane, r = L / CPR, x = (L % CPR) ^ attn_swz<D>(r);
        const int t = t0 + r;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (__attribute__((address_space(3))) void *)(s_v + u * 512), 16,
            t < a.T ? (t * D + 8 * x) * 2 : kAttnOob, 0, 0, kStreamPolicy);
    }

    __builtin_amdgcn_sched_barrier(0);  // every DMA issued before the first read
    // the single workgroup writes the output after its last barrier
    void *out = nullptr;
    int32_t out_bf16 = 0;
    if constexpr (W > 1) {
        out = hold_sgpr(a.out);
        out_bf16 = hold_sgpr(a.out_bf16);
    }
    // key rows back as A operands: lane l takes row 16 b + l % 16 at d chunk
    // 4 kk + l / 16
    uint4 ka[NB][KK];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int r = 16 * b + col, X = 4 * kk + grp;
            ka[b][kk] = *reinterpret_cast<const uint4 *>(
                reinterpret_cast<const char *>(s_k) + (r * CPR + (X ^ attn_swz<D>(r))) * 16);
        }
    // 2. scores in base-2 units, -inf past T; the wave's maximum per head
    f32x4_t sc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        sc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, ka[b][kk]), __builtin_bit_cast(bf16x8_t, qb[kk]),
                sc[b], 0, 0, 0);
    }
    float m = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 16 * b + 4 * grp + r;
            sc[b][r] = t < a.T ? sc[b][r] * a.scale2 : -INFINITY;
            m = fmaxf(m, sc[b][r]);
        }
    {
        const uint32_t b16 = __builtin_bit_cast(uint32_t, m);
        const f32x2_t r16 = __builtin_bit_cast(
            f32x2_t, __builtin_amdgcn_permlane16_swap(b16, b16, false, false));
        m = fmaxf(r16.x, r16.y);
        const uint32_t b32 = __builtin_bit_cast(uint32_t, m);
        const f32x2_t r32 = __builtin_bit_cast(
            f32x2_t, __builtin_amdgcn_permlane32_swap(b32, b32, false, false));
        m = fmaxf(r32.x, r32.y);
    }

    // 3. p = exp2(s - max) (0 past T), its sum, and the hi / lo A operands
    //    (a chunk of the split starts below T; a wave of a single workgroup
    //    whose positions all lie past T has max -inf and takes p = 0)
    const float mref = (W > 1 && m == -INFINITY) ? 0.0f : m;
    float l = 0.0f;
    bf16x8_t ph[NB / 2], pl[NB / 2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(sc[b][r] - mref);
            l += p;
            const __bf16 hi = (__bf16)p;
            ph[b / 2][(b & 1) * 4 + r] = hi;
            pl[b / 2][(b & 1) * 4 + r] = (__bf16)(p - (float)hi);
        }
    l = sum_xor32(sum_xor16(l));

    // 4. O = P V per 16-column tile, V through transposing LDS reads
    //    (source lane 4j + a of group q: row 4q + j of the block, columns
    //    4a .. 4a+3 of the tile)
    const int vj = (lane >> 2) & 3, va = lane & 3;
    f32x4_t o[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
        o[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const int X = 2 * dt + (va >> 1);
#pragma unroll
        for (int mm = 0; mm < NB / 2; ++mm) {
            i16x4_t h[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = 32 * mm + 16 * e + 4 * grp + vj;
                const int off = (r * CPR + (X ^ attn_swz<D>(r))) * 16 + (va & 1) * 8;
                h[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(
                        (__attribute__((address_space(3))) char *)s_v + off));
            }
            const bf16x8_t vb = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[mm], vb, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[mm], vb, o[dt], 0, 0, 0);
        }
    }

    if constexpr (W > 1) {
        // 5'. single workgroup: merge the waves in LDS and write the output
        if (lane < 16) {
            s_ml[wave][0][lane] = m;
            s_ml[wave][1][lane] = l;
        }
        if (wave > 0)
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) s_o[wave - 1][dt][lane] = o[dt];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        if (wave > 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = 4 * grp + r;
            float M = s_ml[0][0][head];
#pragma unroll
            for (int w = 1; w < W; ++w) M = fmaxf(M, s_ml[w][0][head]);
            float L = 0.0f, f[W];
#pragma unroll
            for (int w = 0; w < W; ++w) {
                f[w] = __builtin_amdgcn_exp2f(s_ml[w][0][head] - M);  // 0 for an empty wave
                L = fmaf(s_ml[w][1][head], f[w], L);
            }
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) {
                float v = o[dt][r] * f[0];
#pragma unroll
                for (int w = 1; w < W; ++w) v = fmaf(s_o[w - 1][dt][lane][r], f[w], v);
                if (head < G)
                    store_out(out, (int64_t)(g * G + head) * D + dt * 16 + col, v / L,
                              out_bf16);
            }
        }
        return;
    }

    // 5. the chunk's partial sums: lane (column c, group q) holds heads
    //    4q .. 4q+3 of columns dt * 16 + c
    const int64_t slot = (int64_t)g * a.nchunks + c;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = 4 * grp + r;
            if (head < G) a.part[(slot * G + head) * D + dt * 16 + col] = o[dt][r];
        }
    if (lane < G) {
        a.ml[(slot * G + lane) * 2] = m;
        a.ml[(slot * G + lane) * 2 + 1] = l;
    }
}

// Wave-wide maximum / sum: DPP butterflies inside each row of 16 lanes (quad
// swaps, half-row and row mirrors), then the two row swaps.  Every lane ends
// with the same bits.  All 64 lanes must be active.
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                            0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                            0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                            0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                            0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    const uint32_t b16 = __builtin_bit_cast(uint32_t, v);
    const f32x2_t r16 =
        __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane16_swap(b16, b16, false, false));
    v = op(r16.x, r16.y);
    const uint32_t b32 = __builtin_bit_cast(uint32_t, v);
    const f32x2_t r32 =
        __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane32_swap(b32, b32, false, false));
    return op(r32.x, r32.y);
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce<true>(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<false>(v); }

// One wave per (query head h = g * G + i, 16 output columns).  Rounds of 64
// chunks: lane k takes chunk c0 + k's (max, sum), and the wave maximum gives
// every chunk's factor exp2(m_c - M); lane (phase c, column group q), lane =
// 4c + q, takes columns 4q .. 4q+3 of chunks 16u + c (four 16-byte loads,
// all issued before the first use), gets each chunk's factor from the
// chunk's lane by ds_bpermute, and the 16 phases are added in a fixed order
// (within each row of 16 lanes by rotates of 4 and 8 lanes, then across rows
// by lane pairs 16 apart and 32 apart).  Each round rescales the running
// sums to the new maximum.  No LDS and no barrier.  Narrow column slices
// give four times the waves of 64-column ones, and each issues a quarter of
// the loads.
constexpr int kCombineCols = 16;
template <int D, int G>
__global__ __launch_bounds__(64) void k_attn_combine(const uint16_t *q, const uint16_t *k,
                                                     const uint16_t *v, float *part, float *ml,
                                                     int32_t tcap, int32_t T, int32_t nchunks,
                                                     float scale2, AttnArgs cold) {
    constexpr int NG = kCombineCols / 4, PH = 64 / NG;  // column groups, chunk phases
    const AttnArgs a = attn_hot_args(cold, q, k, v, part, ml, tcap, T, nchunks, scale2);
    const int h = blockIdx.x, lane = threadIdx.x;
    const int g = h / G, i = h - g * G;
    const int e0 = blockIdx.y * kCombineCols + (lane % NG) * 4, ph = lane / NG;
    const int nc = a.nchunks;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (int64_t)g * nc * G * D, 0, nc * G * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
        a.ml + (int64_t)g * nc * G * 2, 0, nc * G * 2 * 4, 0x00020000);
    float M = -INFINITY, L = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const int n = min(64, nc - c0);
        const f32x2_t ml = __builtin_bit_cast(
            f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                         mr, lane < n ? ((c0 + lane) * G + i) * 8 : kAttnOob, 0, 0));
        f32x4_t pv[64 / PH];
#pragma unroll
        for (int u = 0; u < 64 / PH; ++u) {
            const int cu = PH * u + ph;
            pv[u] = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                             pr, cu < n ? (((c0 + cu) * G + i) * D + e0) * 4 : kAttnOob, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);
        const float m = lane < n ? ml.x : -INFINITY;
        const float Mn = fmaxf(M, wave_max(m));
        const float f = lane < n ? __builtin_amdgcn_exp2f(m - Mn) : 0.0f;
        const float r = __builtin_amdgcn_exp2f(M - Mn);  // 0 on the first round
        L = fmaf(L, r, wave_sum(lane < n ? ml.y * f : 0.0f));
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 64 / PH; ++u) {
            const float fu = __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute((PH * u + ph) * 4, __builtin_bit_cast(int, f)));
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(pv[u][j], fu, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // the four phases of a row (lanes 4 apart), then the four rows
            float t = acc[j];
            t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                               0, __builtin_bit_cast(int, t), 0x124, 0xF, 0xF, false));
            t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                               0, __builtin_bit_cast(int, t), 0x128, 0xF, 0xF, false));
            o[j] = fmaf(o[j], r, sum_xor32(sum_xor16(t)));
        }
        M = Mn;
    }
    if (ph == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j) store_out(a.out, (int64_t)h * D + e0 + j, o[j] / L, a.out_bf16);
}

namespace {

// Positions per chunk: kAttnChunk for the one-launch path and for long
// contexts; half of it for the split at mid contexts (at most kAttnMidT
// positions), where twice the workgroups fill the chip better than the
// extra partials cost (measured crossover between 2048 and 4096).
constexpr int64_t kAttnMidT = 2048;
int attn_chunk(int64_t d, int64_t T) {
    const bool single = ceil_div(T, kAttnChunk) <= 256 / d;
    return (!single && T <= kAttnMidT) ? kAttnChunk / 2 : kAttnChunk;
}

int64_t attn_chunks(int64_t d, int64_t T) { return ceil_div(T, attn_chunk(d, T)); }

// Launch one attention kernel: the preloaded leading parameters, then the
// whole struct.
template <typename Kern>
tt_status launch_attn(const char *what, Kern kernel, dim3 grid, dim3 block, hipStream_t s,
                      const AttnArgs &a) {
    return launch(what, kernel, grid, block, 0, s, a.q, a.k, a.v, a.part, a.ml, a.tcap, a.T,
                  a.nchunks, a.scale2, a);
}

template <int D, int G>
tt_status launch_attn(const AttnArgs &a, hipStream_t s) {
    constexpr int W = attn_single_waves<D>();
    constexpr int NB = kAttnChunk / 16;
    const bool full = attn_chunk(D, a.T) == kAttnChunk;
    if (full && a.nchunks <= W)
        return launch_attn("gqa attention (single workgroup)", k_attn_partial<D, G, NB, W>,
                           dim3(1u, (unsigned)a.hkv), dim3(64 * W), s, a);
    if (full)
        TT_TRY(launch_attn("gqa attention (chunks)", k_attn_partial<D, G, NB, 1>,
                           dim3((unsigned)a.nchunks, (unsigned)a.hkv), dim3(64), s, a));
    else
        TT_TRY(launch_attn("gqa attention (chunks)", k_attn_partial<D, G, NB / 2, 1>,
                           dim3((unsigned)a.nchunks, (unsigned)a.hkv), dim3(64), s, a));
    return launch_attn("gqa attention (combine)", k_attn_combine<D, G>,
                       dim3((unsigned)a.hq, (unsigned)(D / kCombineCols)), dim3(64), s, a);
}

template <int D>
tt_status launch_attn_g(const AttnArgs &a, int G, hipStream_t s) {
    switch (G) {
        case 1: return launch_attn<D, 1>(a, s);
        case 2: return launch_attn<D, 2>(a, s);
        case 4: return launch_attn<D, 4>(a, s);
        default: return launch_attn<D, 8>(a, s);
    }
}

tt_status check_attn_shape(int64_t hq, int64_t hkv, int64_t d, int64_t T) {
    TT_TRY(check_range(hkv, 1, 1024, "hkv"));
    TT_TRY(check_range(hq, hkv, 8 * hkv, "hq"));
    if (hq % hkv) return fail(TT_E_SHAPE, "hq = %lld is not a multiple of hkv = %lld",
                              (long long)hq, (long long)hkv);
    const int64_t G = hq / hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(TT_E_SHAPE, "hq / hkv = %lld; 1, 2, 4 or 8 is supported", (long long)G);
    if (d != 64 && d != 128) return fail(TT_E_SHAPE, "d = %lld; 64 or 128 is supported",
                                         (long long)d);
    TT_TRY(check_range(T, 1, TT_MAX_ATTN_T, "T"));
    return TT_OK;
}

}  // namespace
}  // namespace tt

using namespace tt;

extern "C" int64_t tt_gqa_attention_workspace_bytes(int64_t hq, int64_t hkv, int64_t d,
                                                    int64_t T) {
    tt_status st = check_attn_shape(hq, hkv, d, T);
    if (st != TT_OK) return st;
    return hq * attn_chunks(d, T) * (d + 2) * 4;
}

namespace tt {
namespace {

// The checks and launches of one attention call, its per-chunk partials in
// `workspace` (device memory of workspace_bytes).
tt_status attn_decode(const void *q, const void *k_cache, const void *v_cache, int64_t hq,
                      int64_t hkv, int64_t d, int64_t tcap, int64_t T, float scale, void *out,
                      int32_t out_dtype, void *workspace, int64_t workspace_bytes,
                      void *stream) {
    TT_TRY(check_ptr(q, "q"));
    TT_TRY(check_ptr(k_cache, "k_cache"));
    TT_TRY(check_ptr(v_cache, "v_cache"));
    TT_TRY(check_ptr(out, "out"));
    TT_TRY(check_ptr(workspace, "workspace"));
    TT_TRY(check_attn_shape(hq, hkv, d, T));
    TT_TRY(check_range(tcap, T, TT_MAX_ATTN_T, "tcap"));
    TT_TRY(check_dtype(out_dtype, "out_dtype"));
    TT_TRY(check_align(q, 16, "q"));
    TT_TRY(check_align(k_cache, 16, "k_cache"));
    TT_TRY(check_align(v_cache, 16, "v_cache"));
    TT_TRY(check_align(workspace, 16, "workspace"));
    TT_TRY(check_align(out, out_dtype == TT_F32 ? 4 : 2, "out"));
    const int64_t need = tt_gqa_attention_workspace_bytes(hq, hkv, d, T);
    if (workspace_bytes < need)
        return fail(TT_E_SIZE, "workspace holds %lld bytes, the call needs %lld",
                    (long long)workspace_bytes, (long long)need);
    if ((int64_t)hkv * tcap * d * 2 > (int64_t)INT32_MAX)
        return fail(TT_E_SHAPE, "a kv head's cache exceeds 2 GiB");
    AttnArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k_cache);
    a.v = static_cast<const uint16_t *>(v_cache);
    a.hq = (int32_t)hq;
    a.hkv = (int32_t)hkv;
    a.tcap = (int32_t)tcap;
    a.T = (int32_t)T;
    a.nchunks = (int32_t)attn_chunks(d, T);
    a.scale2 = scale * 1.4426950408889634f;
    const int64_t G = hq / hkv;
    a.part = static_cast<float *>(workspace);
    a.ml = a.part + hq * (int64_t)a.nchunks * d;
    a.out = out;
    a.out_bf16 = out_dtype == TT_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tt_status st = d == 64 ? launch_attn_g<64>(a, (int)G, s) : launch_attn_g<128>(a, (int)G, s);
    if (st == TT_OK) clear_error();
    return st;
}

constexpr int64_t kAttnScratchBytes = TT_ATTN_SCRATCH_BYTES;

}  // namespace

// Partials of the allocation-free entry point: one array per device, held
// until the process ends and shared by every such call on that device.  In
// host code its name is only a stand-in; kernels get its device address,
// looked up once per device.
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

namespace {

std::atomic<void *> g_scratch_addr[64];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (TT_E_HIP if the lookup
// fails); looked up on the first call per device, with that device current.
tt_status scratch_addr(void **ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(TT_E_HIP, "gqa attention (no allocation): no usable current device");
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(TT_E_HIP, "gqa attention (no allocation): scratch lookup failed: %s",
                            hipGetErrorString(e));
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return TT_OK;
}

}  // namespace
}  // namespace tt

extern "C" tt_status tt_gqa_attention_decode(const void *q, const void *k_cache,
                                             const void *v_cache, int64_t hq, int64_t hkv,
                                             int64_t d, int64_t tcap, int64_t T, float scale,
                                             void *out, int32_t out_dtype, void *workspace,
                                             int64_t workspace_bytes, void *stream) {
    return attn_decode(q, k_cache, v_cache, hq, hkv, d, tcap, T, scale, out, out_dtype,
                       workspace, workspace_bytes, stream);
}

extern "C" tt_status tt_gqa_attention_decode_noalloc(const void *q, const void *k_cache,
                                                     const void *v_cache, int64_t hq,
                                                     int64_t hkv, int64_t d, int64_t tcap,
                                                     int64_t T, float scale, void *out,
                                                     int32_t out_dtype, void *stream) {
    TT_TRY(check_attn_shape(hq, hkv, d, T));
    const int64_t need = tt_gqa_attention_workspace_bytes(hq, hkv, d, T);
    if (need > kAttnScratchBytes)
        return fail(TT_E_SIZE, "gqa attention (no allocation): the call needs %lld bytes of "
                    "partials, more than the %lld the library holds per device",
                    (long long)need, (long long)kAttnScratchBytes);
    void *ws = nullptr;
    TT_TRY(scratch_addr(&ws));
    return attn_decode(q, k_cache, v_cache, hq, hkv, d, tcap, T, scale, out, out_dtype, ws,
                       kAttnScratchBytes, stream);
}
