// moe.hip -- routed-expert stages on gfx950: top-k routing and the MXFP4
// down projection with the weighted combine (stardance page, "ThinTensor
// Improvements": exact routing; "numerical drift & speedups": selected-expert
// MXFP4 matvecs; "Dev Log #2": router and expert stages of an MoE model).
//
// Routing: one wave per token.  Each expert's (bf16 logit, index) becomes one
// orderable key; an expert's rank is the number of larger keys, and ranks
// below topk are the selection in descending order, ties to the lower index.
// The weights are the softmax of the selected logits.
// Ids and weights stay on the device for the expert kernels.
//
// Down + combine: one workgroup per (16-row tile of the output, token) with
// topk * S waves -- wave (j, part) streams expert ids[b][j]'s tile over its
// share of the K units against h[b][j] staged in LDS: bf16 h on the scaled
// FP4 x FP8 MFMA (the expert's packed units as A operands, h split into two
// E4M3 parts as B), fp32 h on the vector ALUs.  The per-row partials are
// combined in a fixed order (parts, then slots j = 0..topk-1), so there are
// no atomics and the result is bit-reproducible.
#include <algorithm>

#include "device.h"
#include "tt_internal.h"

namespace tt {

struct RouteArgs {
    const uint16_t *logits;
    int32_t n_exp, topk;
    int32_t *ids;
    float *w;
};

// Orderable 32-bit key of (bf16 logit, expert index): a larger key is a larger
// logit, and among equal logits the lower index.  -0 is folded onto +0 so the
// two compare equal, as the values do.
__device__ __forceinline__ uint32_t route_key(uint32_t bits, int e) {
    bits = (bits == 0x8000u) ? 0u : bits;
    const uint32_t ord = (bits & 0x8000u) ? (~bits & 0xFFFFu) : (bits | 0x8000u);
    return (ord << 16) | (0xFFFFu - (uint32_t)e);
}

// One wave per token.  Every lane writes the keys of its (up to 4) experts to
// LDS, then counts how many keys exceed each of its own: that count is the
// expert's rank, and ranks 0 .. topk-1 are the selection in descending order.
// The selected lanes publish their logits by rank; lane 0 forms the softmax
// over them in rank order.
__global__ __launch_bounds__(64) void k_route_topk(const uint16_t *logits, int32_t n_exp_,
                                                   int32_t topk_, int32_t *ids, float *w) {
    const RouteArgs ra{logits, n_exp_, topk_, ids, w};
    __shared__ uint32_t keys[TT_MAX_EXPERTS];
    __shared__ float selv[TT_MAX_TOPK];
    __shared__ int32_t seli[TT_MAX_TOPK];
    const int n_exp = ra.n_exp, topk = ra.topk;
    const int b = blockIdx.x, lane = threadIdx.x;
    const uint16_t *lb = ra.logits + (int64_t)b * n_exp;
    uint32_t raw[4], key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = lb[min(lane + 64 * i, n_exp - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        key[i] = route_key(raw[i], e);
        if (e < n_exp) keys[e] = key[i];
    }
    __syncthreads();
    int rank[4] = {0, 0, 0, 0};
    for (int e = 0; e < n_exp; ++e) {
        const uint32_t k = keys[e];
#pragma unroll
        for (int i = 0; i < 4; ++i) rank[i] += k > key[i] ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < n_exp && rank[i] < topk) {
            selv[rank[i]] = bf16_bits_to_f32(raw[i]);
            seli[rank[i]] = e;
        }
    }
    __syncthreads();
    if (lane == 0) {
        const float m = selv[0];
        float den = 0.0f;
        for (int j = 0; j < topk; ++j) den += expf(selv[j] - m);
        for (int j = 0; j < topk; ++j) {
            ra.ids[(int64_t)b * topk + j] = seli[j];
            ra.w[(int64_t)b * topk + j] = expf(selv[j] - m) / den;
        }
    }
}

struct DownArgs {
    const uint8_t *bank;
    int64_t expert_stride, tile_stride;
    int32_t n_experts, hidden, inter;  // output rows = hidden, K = inter
    int32_t nb, units, qv_last, scale_off, ps_off;
    const void *h;                     // [batch][topk][inter]
    const int32_t *ids;
    const float *wt;
    int32_t topk;
    int32_t S;                         // waves per slot (K split)
    int32_t spr;                       // slots per round
    void *y;                           // [batch][hidden]
    int32_t y_bf16;
};

// The argument struct with the leading kernel parameters of the down
// kernels written in: everything read before the weight loads (the tile
// geometry follows from the block count nb, K = inter = 32 nb; an expert's
// pack is ceil(hidden / 16) whole tiles), and the output, which the tail
// after the last barrier needs (read from argument memory there, it would
// add a memory round trip to the end of every call).  The first 14 dwords
// of arguments are preloaded, so topk and the output's bf16 flag share one
// (topk | bf16 << 16).
__device__ __forceinline__ DownArgs down_hot_args(DownArgs a, const uint8_t *bank,
                                                  const void *h, const int32_t *ids, int32_t nb,
                                                  int32_t n_experts, int32_t hidden,
                                                  int32_t topk_yb, int32_t S, int32_t spr,
                                                  void *y) {
    const MxGeom g = mx_geom(32 * (int64_t)nb);
    a.bank = bank;
    a.h = h;
    a.ids = ids;
    a.nb = nb;
    a.inter = 32 * nb;
    a.units = (int32_t)g.units;
    a.qv_last = (int32_t)g.qv_last;
    a.scale_off = (int32_t)g.scale_off;
    a.ps_off = (int32_t)g.ps_off;
    a.tile_stride = g.stride;
    a.n_experts = n_experts;
    a.hidden = hidden;
    a.expert_stride = ceil_div(hidden, kTileRows) * g.stride;
    a.topk = topk_yb & 0xFFFF;
    a.S = S;
    a.spr = spr;
    a.y = y;
    a.y_bf16 = topk_yb >> 16;
    return a;
}

// Tuning: K units (128 elements) per wave.
#ifndef TT_DOWN_UPW
#define TT_DOWN_UPW 8
#endif
constexpr int kDownOob = 0x7FFFFF00;

// Orders a wave's own LDS writes before its later LDS reads (the hardware
// completes one wave's LDS accesses in order; this keeps the compiler from
// moving them across).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ void down_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The combine after the down kernels' last barrier, run by all 64 lanes of
// one wave: row r's output is the sum over slots j of w_j (ps_j[r] dot_j[r]),
// dot_j = the slot's S partial rows summed in part order.  Lane (r = lane %
// 16, quarter q = lane / 16) takes slots q and q + 4; it reads all parts of
// a slot at once (indexes clamped into the table, the surplus masked off)
// rather than one LDS round trip per part.  The quarters are then added as
// (q0 + q1) + (q2 + q3) by lane swaps: a fixed order, the same bits on every
// run.  A bad expert id's NaN weight makes the row NaN.
static_assert(TT_MAX_TOPK <= 8, "two slots per quarter of the wave");
template <int SMAX>
__device__ __forceinline__ float down_combine_rows_n(const float *red, const float *pss, int topk,
                                                     int S, int lane) {
    const int r = lane & 15, q = lane >> 4;
    float acc = 0.0f;
#pragma unroll
    for (int jq = 0; jq < 2; ++jq) {
        if (4 * jq >= topk) break;  // uniform: slots 4.. only when topk > 4
        const int jj = q + 4 * jq, jc = min(jj, topk - 1);
        float v[SMAX];  // S <= SMAX parts
#pragma unroll
        for (int pp = 0; pp < SMAX; ++pp) v[pp] = red[(jc * S + min(pp, S - 1)) * 16 + r];
        float dot = v[0];
#pragma unroll
        for (int pp = 1; pp < SMAX; ++pp) dot = pp < S ? dot + v[pp] : dot;
        const float t = pss[jc * 17 + 16] * (pss[jc * 17 + r] * dot);
        if (jj < topk) acc = jq == 0 ? t : acc + t;
    }
    return sum_xor32(sum_xor16(acc));
}
__device__ __forceinline__ float down_combine_rows(const float *red, const float *pss, int topk,
                                                   int S, int lane) {
    return S <= 4 ? down_combine_rows_n<4>(red, pss, topk, S, lane)
                  : down_combine_rows_n<16>(red, pss, topk, S, lane);
}

// fp32 h (vector ALUs; bf16 h takes the scaled-MFMA kernel below).  One
// workgroup per (16-row output tile, token).  Slots are processed in rounds
// of spr; within a round wave (slot j, part p) owns units
// [p * UPW, p * UPW + UPW) of expert ids[b][j]'s tile.  Issue order per wave:
// its share of the round's activations, then each scale dword followed by its
// four code units, then the postscales.  A slot with a bad expert id gets a
// zero-length buffer descriptor, so its loads read nothing and return zeros.
template <int UPW>
__global__ __launch_bounds__(1024) void k_down_combine(const uint8_t *bank, const void *h,
                                                  const int32_t *__restrict__ ids, int32_t nb,
                                                  int32_t n_experts, int32_t hidden, int32_t topk_yb,
                                                  int32_t S_, int32_t spr_, void *out,
                                                  DownArgs cold) {
    const DownArgs a = down_hot_args(cold, bank, h, ids, nb, n_experts, hidden, topk_yb, S_, spr_, out);
    static_assert(UPW % 4 == 0 && UPW <= 16, "units per wave");
    constexpr int ESZ = 4;                       // fp32 h
    constexpr int XC = UPW * ESZ / 8;            // 16-byte chunks per thread per round
    extern __shared__ __align__(16) uint8_t smem[];
    const int S = a.S, topk = a.topk, spr = a.spr;
    const int kp = S * UPW * 128;                // staged K per slot, zero past inter
    const int slot_chunks = kp * ESZ / 16;
    uint4 *xs4 = reinterpret_cast<uint4 *>(smem);
    float *red = reinterpret_cast<float *>(smem + (size_t)spr * kp * ESZ);  // [topk][S][16]
    float *pss = red + topk * S * 16;                                       // [topk][17]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = blockIdx.x, b = blockIdx.y;
    const int q = lane >> 4;
    const int js = wave / S, part = wave - js * S;
    const int valid_chunks = a.inter * ESZ / 16;
    const uint4 *hsrc = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.h) +
                                                        (size_t)b * topk * a.inter * ESZ);

    for (int jb = 0; jb < topk; jb += spr) {
        const int j = jb + js;
        const bool slot_ok = j < topk;
        // 1. the activations this wave's units read: slot j, chunks
        //    part * UPW * 32 + c * 64 + lane (4 fp32 each); issued before
        //    the expert id, whose wait they then overlap (the id is a scalar
        //    load, counted apart from these vector loads)
        const int cw0 = part * UPW * 32;
        uint4 hv[XC];
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int ci = cw0 + c * 64 + lane;
            hv[c] = (slot_ok && ci < valid_chunks) ? hsrc[j * valid_chunks + ci]
                                                  : make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int e = slot_ok ? ids[b * topk + j] : -1;
        const bool valid = e >= 0 && e < a.n_experts;

        // 2. weights
        const uint8_t *tb = valid ? a.bank + (int64_t)e * a.expert_stride +
                                        (int64_t)tile * a.tile_stride
                                  : a.bank;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(tb), 0, valid ? (int)a.tile_stride : 0, 0x00020000);
        const int u0 = part * UPW;
        const int n = max(0, min(UPW, a.units - u0));
        uint4 c[UPW];
        uint32_t sd[UPW / 4];
        const int voff = u0 * kUnitBytes + lane * 16;
        const int soff = a.scale_off + (u0 >> 2) * kGroupBytes + lane * 4;
#pragma unroll
        for (int g = 0; g < UPW / 4; ++g) {
            sd[g] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, 4 * g < n ? soff + g * kGroupBytes : kDownOob, 0, kStreamPolicy);
#pragma unroll
            for (int i = 4 * g; i < 4 * g + 4; ++i) {
                const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, i < n ? voff + i * kUnitBytes : kDownOob, 0, kStreamPolicy);
                c[i] = make_uint4(v.x, v.y, v.z, v.w);
            }
        }
        const float ps = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       rs, (part == 0 && lane < 16) ? a.ps_off + lane * 4 : kDownOob, 0,
                       kStreamPolicy));
        const float wj = slot_ok ? a.wt[b * topk + j] : 0.0f;

        // 3. activations to the wave's own part of LDS (only this wave reads
        //    it, in this round and the next: a wave's LDS accesses complete
        //    in order, so no barrier)
#pragma unroll
        for (int cc = 0; cc < XC; ++cc) xs4[js * slot_chunks + cw0 + cc * 64 + lane] = hv[cc];
        wave_lds_fence();

        // 4. consume the units in load order
        float acc = 0.0f;
        const float4 *xb = reinterpret_cast<const float4 *>(smem) +
                           ((size_t)js * kp + (4 * u0 + q) * 32) / 4;
#pragma unroll
        for (int i = 0; i < UPW; ++i)
            acc = fmaf(fp4x32_dot_f32(c[i], xb + i * 32),
                       e8m0_f32((sd[i >> 2] >> (8 * (i & 3))) & 255u), acc);
        acc = sum_xor32(sum_xor16(acc));
        if (slot_ok) {
            if (lane < 16) red[(j * S + part) * 16 + lane] = acc;
            if (part == 0 && lane < 16) pss[j * 17 + lane] = ps;
            if (part == 0 && lane == 16) pss[j * 17 + 16] = valid ? wj : __builtin_nanf("");
        }
    }
    down_lds_barrier();
    if (wave != 0) return;
    const float y = down_combine_rows(red, pss, topk, S, lane);
    const int row = tile * 16 + lane;
    if (lane < 16 && row < a.hidden) store_out(a.y, (int64_t)b * a.hidden + row, y, a.y_bf16);
}

// Scaled-MFMA form of the same kernel for bf16 h: each unit goes to
// v_mfma_scale_f32_16x16x128_f8f6f4 with the expert's packed unit and its
// E8M0 bytes as the A operand and the slot's h, split per 32-element block
// into two E4M3 parts (device.h), as B column 0 (hi) and column 8 (lo).
// LDS: the parts [spr][2][kp] bytes, their scale bytes [spr][2][4][kp/128],
// 32 zero bytes (B of the unused columns), then the partial rows and the
// postscales / weights of the combine.
template <int UPW>
__global__ __launch_bounds__(1024) void k_down_mx(const uint8_t *bank, const void *h,
                                                  const int32_t *__restrict__ ids, int32_t nb,
                                                  int32_t n_experts, int32_t hidden, int32_t topk_yb,
                                                  int32_t S_, int32_t spr_, void *out,
                                                  DownArgs cold) {
    const DownArgs a = down_hot_args(cold, bank, h, ids, nb, n_experts, hidden, topk_yb, S_, spr_, out);
    static_assert(UPW % 4 == 0 && UPW <= 16, "units per wave");
    constexpr int XC = UPW / 4;                  // 16-byte chunks per thread per round
    extern __shared__ __align__(16) uint8_t smem[];
    const int S = a.S, topk = a.topk, spr = a.spr;
    const int kp = S * UPW * 128;                // staged K per slot, zero past inter
    const int kpu = kp / 128;
    const int qsz = spr * 2 * kp, zoff = qsz + spr * kp / 16;
    float *red = reinterpret_cast<float *>(smem + zoff + 32);  // [topk][S][16]
    float *pss = red + topk * S * 16;                          // [topk][17]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = blockIdx.x, b = blockIdx.y;
    const int js = wave / S, part = wave - js * S;
    const int valid_chunks = a.inter / 8;
    const uint4 *hsrc = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.h) +
                                                        (size_t)b * topk * a.inter);
    const int col = lane & 15, grp = lane >> 4, hl = col >> 3;
    const bool bact = (col & 7) == 0;            // columns 0 (hi) and 8 (lo)

    for (int jb = 0; jb < topk; jb += spr) {
        const int j = jb + js;
        const bool slot_ok = j < topk;
        // 1. the activations this wave's units read: slot j, chunks
        //    part * UPW * 16 + c * 64 + lane (8 bf16 each); issued before
        //    the expert id, whose wait they then overlap (the id is a scalar
        //    load, counted apart from these vector loads)
        const int cw0 = part * UPW * 16;
        uint4 hv[XC];
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int ci = cw0 + c * 64 + lane;
            hv[c] = (slot_ok && ci < valid_chunks) ? hsrc[j * valid_chunks + ci]
                                                  : make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int e = slot_ok ? ids[b * topk + j] : -1;
        const bool valid = e >= 0 && e < a.n_experts;

        // 2. weights
        const uint8_t *tb = valid ? a.bank + (int64_t)e * a.expert_stride +
                                        (int64_t)tile * a.tile_stride
                                  : a.bank;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(tb), 0, valid ? (int)a.tile_stride : 0, 0x00020000);
        const int u0 = part * UPW;
        const int n = max(0, min(UPW, a.units - u0));
        uint4 c[UPW];
        uint32_t sd[UPW / 4];
        const int voff = u0 * kUnitBytes + lane * 16;
        const int soff = a.scale_off + (u0 >> 2) * kGroupBytes + lane * 4;
#pragma unroll
        for (int g = 0; g < UPW / 4; ++g) {
            sd[g] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, 4 * g < n ? soff + g * kGroupBytes : kDownOob, 0, kStreamPolicy);
#pragma unroll
            for (int i = 4 * g; i < 4 * g + 4; ++i) {
                const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, i < n ? voff + i * kUnitBytes : kDownOob, 0, kStreamPolicy);
                c[i] = make_uint4(v.x, v.y, v.z, v.w);
            }
        }
        const float ps = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       rs, (part == 0 && lane < 16) ? a.ps_off + lane * 4 : kDownOob, 0,
                       kStreamPolicy));
        const float wj = slot_ok ? a.wt[b * topk + j] : 0.0f;
        __builtin_amdgcn_sched_barrier(0);

        // 3. activations -> E4M3 parts in the wave's own part of LDS (only
        //    this wave reads it, in this round and the next; every wave
        //    writes the same zeros to the shared zero slot before it reads
        //    it; a wave's LDS accesses complete in order, so no barrier)
#pragma unroll
        for (int cc = 0; cc < XC; ++cc) {
            const int ci = cw0 + cc * 64 + lane;
            uint2 hi, lo;
            const uint32_t sh = split_chunk(hv[cc], &hi, &lo);
            *reinterpret_cast<uint2 *>(smem + (js * 2) * kp + ci * 8) = hi;
            *reinterpret_cast<uint2 *>(smem + (js * 2 + 1) * kp + ci * 8) = lo;
            if ((ci & 3) == 0) {
                const int blk = ci >> 2;
                smem[qsz + ((js * 2) * 4 + (blk & 3)) * kpu + (blk >> 2)] = (uint8_t)sh;
                smem[qsz + ((js * 2 + 1) * 4 + (blk & 3)) * kpu + (blk >> 2)] = (uint8_t)(sh - 4u);
            }
        }
        if (lane < 8) reinterpret_cast<uint32_t *>(smem + zoff)[lane] = 0u;
        wave_lds_fence();

        // 4. the units in load order, one scaled MFMA each
        const int qbase = bact ? (js * 2 + hl) * kp + u0 * 128 + 16 * grp : zoff;
        const int qstep = bact ? 128 : 0, qhalf = bact ? 64 : 16;
        const int sbase = qsz + ((js * 2 + hl) * 4 + grp) * kpu + u0;
        f32x4_t C = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        uint32_t sb = 0x7F7F7F7Fu;
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            if ((i & 3) == 0 && bact) sb = *reinterpret_cast<const uint32_t *>(smem + sbase + i);
            const uint4 b0 = *reinterpret_cast<const uint4 *>(smem + qbase + i * qstep);
            const uint4 b1 = *reinterpret_cast<const uint4 *>(smem + qbase + i * qstep + qhalf);
            const i32x8_t B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                               (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            const i32x8_t A = {(int)c[i].x, (int)c[i].y, (int)c[i].z, (int)c[i].w, 0, 0, 0, 0};
            C = mfma_fp4_fp8(i & 3, A, B, C, sd[i >> 2], sb);
        }
        // 5. lo column 8 onto column 0 (DPP row shift left by 8); lane
        //    (0, g) holds rows 4g .. 4g+3
        const u32x4_t cw = __builtin_bit_cast(u32x4_t, C);
        f32x4_t y;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            y[r] = C[r] + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                        0, (int)cw[r], 0x108, 0xF, 0xF, false));
        if (slot_ok) {
            if (col == 0) *reinterpret_cast<f32x4_t *>(red + (j * S + part) * 16 + 4 * grp) = y;
            if (part == 0 && lane < 16) pss[j * 17 + lane] = ps;
            if (part == 0 && lane == 16) pss[j * 17 + 16] = valid ? wj : __builtin_nanf("");
        }
    }
    down_lds_barrier();
    if (wave != 0) return;
    const float y = down_combine_rows(red, pss, topk, S, lane);
    const int row = tile * 16 + lane;
    if (lane < 16 && row < a.hidden) store_out(a.y, (int64_t)b * a.hidden + row, y, a.y_bf16);
}

}  // namespace tt

namespace tt {
namespace {

template <int UPW>
tt_status launch_down_mx(const DownArgs &a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
    if (lds > 64 * 1024) TT_TRY((raise_lds_limit<k_down_mx<UPW>>("moe down + combine")));
    return launch("moe down + combine (scaled MFMA)", k_down_mx<UPW>, grid, block, lds, s, a.bank, a.h, a.ids, a.nb,
                  a.n_experts, a.hidden, a.topk | (a.y_bf16 << 16), a.S, a.spr, a.y, a);
}

template <int UPW>
tt_status launch_down(const DownArgs &a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
    if (lds > 64 * 1024) TT_TRY((raise_lds_limit<k_down_combine<UPW>>("moe down + combine")));
    return launch("moe down + combine", k_down_combine<UPW>, grid, block, lds, s, a.bank, a.h, a.ids, a.nb,
                  a.n_experts, a.hidden, a.topk | (a.y_bf16 << 16), a.S, a.spr, a.y, a);
}

}  // namespace
}  // namespace tt

using namespace tt;

extern "C" tt_status tt_moe_route_topk(const void *logits, int64_t batch, int64_t n_experts,
                                       int64_t topk, int32_t *ids, float *w, void *stream) {
    TT_TRY(check_ptr(logits, "logits"));
    TT_TRY(check_ptr(ids, "ids"));
    TT_TRY(check_ptr(w, "w"));
    TT_TRY(check_range(batch, 1, TT_MAX_BATCH, "batch"));
    TT_TRY(check_range(n_experts, 1, TT_MAX_EXPERTS, "n_experts"));
    TT_TRY(check_range(topk, 1, n_experts < TT_MAX_TOPK ? n_experts : TT_MAX_TOPK, "topk"));
    TT_TRY(check_align(logits, 2, "logits"));
    TT_TRY(check_align(ids, 4, "ids"));
    TT_TRY(check_align(w, 4, "w"));
    RouteArgs ra{static_cast<const uint16_t *>(logits), (int32_t)n_experts, (int32_t)topk, ids, w};
    tt_status st = launch("moe route top-k", k_route_topk, dim3((unsigned)batch), dim3(64), 0,
                          static_cast<hipStream_t>(stream), ra.logits, ra.n_exp, ra.topk, ra.ids,
                          ra.w);
    if (st == TT_OK) clear_error();
    return st;
}

extern "C" tt_status tt_moe_mxfp4_down_combine(const void *down_bank, int64_t n_experts,
                                               int64_t hidden, int64_t inter, const void *h,
                                               int32_t h_dtype, const int32_t *ids,
                                               const float *w, int64_t batch, int64_t topk,
                                               void *y, int32_t y_dtype, void *stream) {
    TT_TRY(check_ptr(down_bank, "down_bank"));
    TT_TRY(check_ptr(h, "h"));
    TT_TRY(check_ptr(ids, "ids"));
    TT_TRY(check_ptr(w, "w"));
    TT_TRY(check_ptr(y, "y"));
    TT_TRY(check_range(n_experts, 1, TT_MAX_EXPERTS, "n_experts"));
    TT_TRY(check_range(hidden, 1, TT_MAX_ROWS, "hidden"));
    TT_TRY(check_range(inter, 32, TT_MAX_K, "inter"));
    if (inter % 32) return fail(TT_E_SHAPE, "inter = %lld is not a multiple of 32", (long long)inter);
    TT_TRY(check_range(batch, 1, TT_MAX_BATCH, "batch"));
    TT_TRY(check_range(topk, 1, n_experts < TT_MAX_TOPK ? n_experts : TT_MAX_TOPK, "topk"));
    TT_TRY(check_dtype(h_dtype, "h_dtype"));
    TT_TRY(check_dtype(y_dtype, "y_dtype"));
    TT_TRY(check_align(down_bank, 16, "down_bank"));
    TT_TRY(check_align(h, 16, "h"));
    TT_TRY(check_align(ids, 4, "ids"));
    TT_TRY(check_align(w, 4, "w"));
    TT_TRY(check_align(y, y_dtype == TT_F32 ? 4 : 2, "y"));
    const MxGeom g = mx_geom(inter);
    DownArgs a;
    a.bank = static_cast<const uint8_t *>(down_bank);
    a.tile_stride = g.stride;
    a.expert_stride = ceil_div(hidden, kTileRows) * g.stride;
    a.n_experts = (int32_t)n_experts;
    a.hidden = (int32_t)hidden;
    a.inter = (int32_t)inter;
    a.nb = (int32_t)g.nb;
    a.units = (int32_t)g.units;
    a.qv_last = (int32_t)g.qv_last;
    a.scale_off = (int32_t)g.scale_off;
    a.ps_off = (int32_t)g.ps_off;
    a.h = h;
    a.ids = ids;
    a.wt = w;
    a.topk = (int32_t)topk;
    a.y = y;
    a.y_bf16 = y_dtype == TT_BF16;
    // waves per slot S = ceil(units / UPW) <= 16 (inter <= TT_MAX_K gives at
    // most 128 units), slots per round so that a workgroup holds at most 16
    // waves
    int upw = TT_DOWN_UPW;
    while (ceil_div(g.units, upw) > 16) upw += 4;
    if (upw > 8) return fail(TT_E_SHAPE, "inter = %lld is too long", (long long)inter);
    a.S = (int32_t)ceil_div(g.units, upw);
    a.spr = (int32_t)std::max<int64_t>(1, std::min<int64_t>(topk, 16 / a.S));
    dim3 grid((unsigned)ceil_div(hidden, kTileRows), (unsigned)batch);
    dim3 block((unsigned)(64 * a.S * a.spr));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (h_dtype == TT_BF16) {
        // scaled MFMA: E4M3 parts + scale bytes + zero bytes + partials
        const size_t kp = (size_t)a.S * upw * 128;
        const size_t lds = (size_t)a.spr * 2 * kp + (size_t)a.spr * kp / 16 + 32 +
                           (size_t)topk * a.S * 64 + (size_t)topk * 17 * 4;
        if (lds > 160 * 1024)
            return fail(TT_E_SHAPE, "inter = %lld: the staged activations do not fit in LDS",
                        (long long)inter);
        const tt_status st = upw == 4 ? launch_down_mx<4>(a, grid, block, lds, s)
                                      : launch_down_mx<8>(a, grid, block, lds, s);
        if (st == TT_OK) clear_error();
        return st;
    }
    // fp32 h on the vector ALUs
    const size_t lds = (size_t)a.spr * a.S * upw * 128 * 4 + (size_t)topk * a.S * 64 +
                       (size_t)topk * 17 * 4;
    if (lds > 160 * 1024)
        return fail(TT_E_SHAPE, "inter = %lld: the staged activations do not fit in LDS",
                    (long long)inter);
    tt_status st;
    st = upw == 4 ? launch_down<4>(a, grid, block, lds, s) : launch_down<8>(a, grid, block, lds, s);
    if (st == TT_OK) clear_error();
    return st;
}

