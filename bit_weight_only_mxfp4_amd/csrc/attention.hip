// attention.hip -- single-token grouped-query attention over a bf16 KV cache
// (kerbin.cskartikey.dev/@satvikhardat, "Dev Log #3 -- SmolLM3-3B Results":
// each query head h reads kv head h / (hq / hkv); a score is the key . query
// dot product times the scale; the output is the softmax-weighted sum of the
// values over the cached positions).
//
// Split over positions (flash-decoding style), two kernels:
//  1. k_attn_partial, one workgroup of 4 waves per (64-position chunk, kv
//     head): every wave issues its query slices, then the key rows and value
//     rows of its 16 positions (straight-line buffer loads; positions past T
//     read zeros and score -inf), scores the G query heads of the kv head
//     with dot2 on bf16 pairs, takes the chunk's per-head maximum across the
//     waves, and accumulates p = exp(s - max) and p * V in fp32 (scores are
//     kept in base-2 units, s * log2(e), so each exponential is one
//     v_exp_f32).  The chunk's (max, sum p, sum p V) per head go to the
//     caller's workspace.
//  2. k_attn_combine, one workgroup per query head: rescales the chunks to
//     the global maximum and sums them in chunk order (fixed order: the
//     result is the same on every run).
// Lane mapping: a key/value row of D bf16 is D / 8 lanes x 16 bytes; a wave
// load covers 64 / (D / 8) positions.
#include "device.h"
#include "tt_internal.h"

namespace tt {

#ifndef TT_ATTN_WAVES
#define TT_ATTN_WAVES 4
#endif
#ifndef TT_ATTN_CHUNK
#define TT_ATTN_CHUNK 64
#endif
constexpr int kAttnWaves = TT_ATTN_WAVES;
constexpr int kAttnChunk = TT_ATTN_CHUNK;  // positions per workgroup
constexpr int kAttnPerWave = kAttnChunk / kAttnWaves;
constexpr int kAttnOob = 0x7FFFFF00;

struct AttnArgs {
    const uint16_t *q, *k, *v;  // q [hq][d]; k, v [hkv][tcap][d]
    int32_t hq, hkv, tcap, T, nchunks;
    float scale2;               // scale * log2(e): scores in base-2 units
    float *part;                // [hkv][nchunks][G][D]
    float *ml;                  // [hkv][nchunks][G][2]: chunk max, chunk sum
    void *out;                  // [hq][d]
    int32_t out_bf16;
};

__device__ __forceinline__ uint4 attn_load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void attn_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum / max over the LPT lanes of one position (16 or 8 consecutive lanes)
// with DPP butterflies: quad swaps, then the half-row and row mirrors.
template <int LPT>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(LPT == 8 || LPT == 16, "lanes per position");
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x141, 0xF, 0xF, false));
    if (LPT == 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

template <int D, int G>
__global__ __launch_bounds__(64 * kAttnWaves) void k_attn_partial(AttnArgs a) {
    constexpr int LPT = D / 8;                 // lanes per position
    constexpr int PPL = 64 / LPT;              // positions per wave load
    constexpr int NL = kAttnPerWave / PPL;     // loads per wave for K (and V)
    constexpr int NR = kAttnWaves * PPL;       // position rows per workgroup
    __shared__ float s_max[NR][G];
    __shared__ float s_sum[NR][G];
    __shared__ float s_o[NR][G][D];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x, g = blockIdx.y;
    const int sl = lane % LPT, pg = lane / LPT;  // d-slice, position within a load
    const int t0 = c * kAttnChunk + wave * kAttnPerWave;

    // 1. query slices of the G heads, then the key and value rows
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.q + (int64_t)g * G * D), 0, G * D * 2, 0x00020000);
    uint4 qv[G];
#pragma unroll
    for (int i = 0; i < G; ++i) qv[i] = attn_load16(qr, (i * D + sl * 8) * 2);
    const int64_t head_off = (int64_t)g * a.tcap * D;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.k + head_off), 0, a.T * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.v + head_off), 0, a.T * D * 2, 0x00020000);
    uint4 kv[NL], vv[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int t = t0 + j * PPL + pg;
        kv[j] = attn_load16(kr, t < a.T ? (t * D + sl * 8) * 2 : kAttnOob);
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int t = t0 + j * PPL + pg;
        vv[j] = attn_load16(vr, t < a.T ? (t * D + sl * 8) * 2 : kAttnOob);
    }

    // 2. scores: dot2 over the lane's 8 elements, summed over the LPT lanes
    //    of the position (xor-shuffles stay inside the position's lanes)
    float s[NL][G];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kv[j].x), as_bf16x2(qv[i].x),
                                                        0.0f, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kv[j].y), as_bf16x2(qv[i].y), acc,
                                                  false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kv[j].z), as_bf16x2(qv[i].z), acc,
                                                  false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kv[j].w), as_bf16x2(qv[i].w), acc,
                                                  false);
            acc = row_sum<LPT>(acc);
            const int t = t0 + j * PPL + pg;
            s[j][i] = t < a.T ? acc * a.scale2 : -INFINITY;
        }
    }

    // 3. the chunk's maximum per head: over the row's positions in
    //    registers, then over the rows of all waves through LDS
    const int row = wave * PPL + pg;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        float m = s[0][i];
#pragma unroll
        for (int j = 1; j < NL; ++j) m = fmaxf(m, s[j][i]);
        if (sl == 0) s_max[row][i] = m;
    }
    attn_barrier();
    float mx[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        mx[i] = s_max[0][i];
#pragma unroll
        for (int r = 1; r < NR; ++r) mx[i] = fmaxf(mx[i], s_max[r][i]);
    }

    // 4. p = exp(s - max), its sum and p * V in fp32
    float o[G][8], l[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        l[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const uint32_t vw[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vf[2 * e] = bf16_bits_to_f32(vw[e] & 0xFFFFu);
            vf[2 * e + 1] = bf16_bits_to_f32(vw[e] >> 16);
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float p = __builtin_amdgcn_exp2f(s[j][i] - mx[i]);  // 0 past T
            l[i] += p;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[i][e] = fmaf(p, vf[e], o[i][e]);
        }
    }
    // each row's partial sums go to LDS (a row's lanes hold its d-slices)
#pragma unroll
    for (int i = 0; i < G; ++i) {
        float4 *dst = reinterpret_cast<float4 *>(&s_o[row][i][sl * 8]);
        dst[0] = make_float4(o[i][0], o[i][1], o[i][2], o[i][3]);
        dst[1] = make_float4(o[i][4], o[i][5], o[i][6], o[i][7]);
        if (sl == 0) s_sum[row][i] = l[i];
    }
    attn_barrier();

    // 5. fixed-order sum over the rows, to the workspace
    const int64_t slot = (int64_t)g * a.nchunks + c;
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
        const int i = idx / D, e = idx - i * D;
        float v = s_o[0][i][e];
#pragma unroll
        for (int r = 1; r < NR; ++r) v += s_o[r][i][e];
        a.part[slot * G * D + idx] = v;
    }
    if (tid < G) {
        float v = s_sum[0][tid], m = s_max[0][tid];
#pragma unroll
        for (int r = 1; r < NR; ++r) {
            v += s_sum[r][tid];
            m = fmaxf(m, s_max[r][tid]);
        }
        a.ml[(slot * G + tid) * 2] = m;
        a.ml[(slot * G + tid) * 2 + 1] = v;
    }
}

// One workgroup of 256 threads per query head h = g * G + i.  The chunks go
// in rounds of 64: every thread issues its loads for the round at once
// (thread (e, part) takes element e of chunks part, part + S, ...; wave 0
// takes the chunks' (max, sum)), then wave 0 forms the round maximum, the
// factors exp(m_c - M) and the round's sum, and every thread rescales its
// running sum -- one memory round trip per round.  The parts are added in a
// fixed order at the end.
constexpr int kCombThreads = 256;
constexpr int kCombRound = 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

template <int D, int G>
__global__ __launch_bounds__(kCombThreads) void k_attn_combine(AttnArgs a) {
    constexpr int S = kCombThreads / D;     // chunk parts per element
    constexpr int PER = kCombRound / S;     // chunks per thread per round
    __shared__ float fac[kCombRound];
    __shared__ float stat[2];               // round maximum, round sum
    __shared__ float opart[S][D];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int g = h / G, i = h - g * G;
    const int nc = a.nchunks;
    const int e = tid % D, p = tid / D;
    // chunk c of this head: part at ((g * nc + c) * G + i) * D, (max, sum) at
    // ((g * nc + c) * G + i) * 2
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (int64_t)g * nc * G * D, 0, nc * G * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
        a.ml + (int64_t)g * nc * G * 2, 0, nc * G * 2 * 4, 0x00020000);
    float M = -INFINITY, L = 0.0f, o = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += kCombRound) {
        float pv[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = c0 + p + S * u;
            pv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                pr, c < nc ? ((c * G + i) * D + e) * 4 : kAttnOob, 0, 0));
        }
        float m = -INFINITY, l = 0.0f;
        if (tid < kCombRound && c0 + tid < nc) {
            m = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                mr, ((c0 + tid) * G + i) * 8, 0, 0));
            l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                mr, ((c0 + tid) * G + i) * 8 + 4, 0, 0));
        }
        if (tid < kCombRound) {
            const float Mn = fmaxf(M, wave_max(m));
            const float f = c0 + tid < nc ? __builtin_amdgcn_exp2f(m - Mn) : 0.0f;
            fac[tid] = f;
            const float ls = wave_sum(l * f);
            if (tid == 0) {
                stat[0] = Mn;
                stat[1] = ls;
            }
        }
        __syncthreads();
        const float Mn = stat[0];
        const float r = __builtin_amdgcn_exp2f(M - Mn);  // 0 on the first round
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < PER; ++u) acc = fmaf(pv[u], fac[p + S * u], acc);
        o = fmaf(o, r, acc);
        L = fmaf(L, r, stat[1]);
        M = Mn;
        __syncthreads();
    }
    opart[p][e] = o;
    __syncthreads();
    if (p == 0) {
        float v = opart[0][e];
#pragma unroll
        for (int q = 1; q < S; ++q) v += opart[q][e];
        store_out(a.out, (int64_t)h * D + e, v / L, a.out_bf16);
    }
}

namespace {

int64_t attn_chunks(int64_t T) { return ceil_div(T, kAttnChunk); }

template <int D, int G>
tt_status launch_attn(const AttnArgs &a, hipStream_t s) {
    TT_TRY(launch("gqa attention (chunks)", k_attn_partial<D, G>,
                  dim3((unsigned)a.nchunks, (unsigned)a.hkv), dim3(64 * kAttnWaves), 0, s, a));
    return launch("gqa attention (combine)", k_attn_combine<D, G>, dim3((unsigned)a.hq),
                  dim3(kCombThreads), 0, s, a);
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
    return hq * attn_chunks(T) * (d + 2) * 4;
}

extern "C" tt_status tt_gqa_attention_decode(const void *q, const void *k_cache,
                                             const void *v_cache, int64_t hq, int64_t hkv,
                                             int64_t d, int64_t tcap, int64_t T, float scale,
                                             void *out, int32_t out_dtype, void *workspace,
                                             int64_t workspace_bytes, void *stream) {
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
    a.nchunks = (int32_t)attn_chunks(T);
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
