// moe.hip -- routed-expert stages on gfx950: top-k routing and the MXFP4
// down projection with the weighted combine (stardance page, "ThinTensor
// Improvements": exact routing; "numerical drift & speedups": selected-expert
// MXFP4 matvecs; "Dev Log #2": router and expert stages of an MoE model).
//
// Routing: one wave per token.  Each lane holds up to 4 bf16 logits; topk
// rounds of a wave-wide (value, lower-index) maximum pick the experts in
// descending order, and the weights are the softmax of the selected logits.
// Ids and weights stay on the device for the expert kernels.
//
// Down + combine: one workgroup per (16-row tile of the output, token) with
// topk * S waves -- wave (j, part) streams expert ids[b][j]'s tile over its
// share of the K units against h[b][j] staged in LDS.  The per-row partials
// are combined in a fixed order (parts, then slots j = 0..topk-1), so there
// are no atomics and the result is bit-reproducible.
#include "device.h"
#include "tt_internal.h"

namespace tt {

struct RouteArgs {
    const uint16_t *logits;
    int32_t n_exp, topk;
    int32_t *ids;
    float *w;
};

__global__ __launch_bounds__(64) void k_route_topk(RouteArgs ra) {
    const uint16_t *logits = ra.logits;
    const int n_exp = ra.n_exp, topk = ra.topk;
    int32_t *ids = ra.ids;
    float *w = ra.w;
    const int b = blockIdx.x, lane = threadIdx.x;
    const uint16_t *lb = logits + (int64_t)b * n_exp;
    float v[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < n_exp;
        v[i] = live[i] ? bf16_bits_to_f32(lb[e]) : 0.0f;
    }
    float sel[TT_MAX_TOPK];
    int sid[TT_MAX_TOPK];
    for (int j = 0; j < topk; ++j) {
        // best live candidate of this lane (its indices ascend with i)
        float bv = 0.0f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (live[i] && (bi < 0 || v[i] > bv)) {
                bv = v[i];
                bi = lane + 64 * i;
            }
        // wave maximum, ties to the lower index; lanes without a candidate lose
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            const bool take = oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi));
            bv = take ? ov : bv;
            bi = take ? oi : bi;
        }
        sel[j] = bv;
        sid[j] = bi;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == bi) live[i] = false;
    }
    if (lane == 0) {
        const float m = sel[0];
        float den = 0.0f;
        for (int j = 0; j < topk; ++j) den += expf(sel[j] - m);
        for (int j = 0; j < topk; ++j) {
            ids[(int64_t)b * topk + j] = sid[j];
            w[(int64_t)b * topk + j] = expf(sel[j] - m) / den;
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
    int32_t topk, S;
    void *y;                           // [batch][hidden]
    int32_t y_bf16;
};

constexpr int kDownPF = 8;

template <bool HF32>
__global__ __launch_bounds__(1024) void k_down_combine(DownArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int kp = a.units * 128;
    const int esz = HF32 ? 4 : 2;
    float *red = reinterpret_cast<float *>(smem + (size_t)a.topk * kp * esz);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x, b = blockIdx.y;
    const int nthreads = blockDim.x;

    // stage h[b][0..topk-1] (zero-padded to kp each)
    if (HF32) {
        const float4 *src = reinterpret_cast<const float4 *>(
            static_cast<const float *>(a.h) + (int64_t)b * a.topk * a.inter);
        float4 *dst = reinterpret_cast<float4 *>(smem);
        const int per = kp / 4, valid = a.inter / 4;
        for (int i = tid; i < a.topk * per; i += nthreads) {
            const int j = i / per, o = i % per;
            dst[i] = (o < valid) ? src[j * valid + o] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        const uint16_t *src = static_cast<const uint16_t *>(a.h) + (int64_t)b * a.topk * a.inter;
        for (int j = 0; j < a.topk; ++j)
            stage_bf16(reinterpret_cast<uint16_t *>(smem) + j * kp, src + (int64_t)j * a.inter,
                       a.inter, kp, tid, nthreads);
    }
    __syncthreads();

    const int j = wave / a.S, part = wave % a.S;
    const int e = a.ids[b * a.topk + j];
    const bool valid = e >= 0 && e < a.n_experts;
    const int r = lane & 15, q = lane >> 4;
    float acc = 0.0f;
    // postscale of this slot's expert for the tile's rows, fetched up front
    float psj = 0.0f;
    if (valid && part == 0 && lane < 16)
        psj = reinterpret_cast<const float *>(a.bank + (int64_t)e * a.expert_stride +
                                              (int64_t)tile * a.tile_stride + a.ps_off)[lane];
    const float wj = a.wt[b * a.topk + j];
    if (valid) {
        const uint8_t *tb = a.bank + (int64_t)e * a.expert_stride + (int64_t)tile * a.tile_stride;
        const uint8_t *sp = tb + a.scale_off + lane * 4;
        const int upw = (a.units + a.S - 1) / a.S;
        const int u0 = part * upw, u1 = min(a.units, u0 + upw);
        for (int kb = u0; kb < u1; kb += kDownPF) {
            uint4 c[kDownPF];
            uint32_t s[kDownPF];
#pragma unroll
            for (int i = 0; i < kDownPF; ++i) {
                const int kk = kb + i;
                if (kk < u1) {
                    const int off = kk * kUnitBytes +
                                    ((kk == a.units - 1 && q >= a.qv_last) ? r * 16 : lane * 16);
                    c[i] = *reinterpret_cast<const uint4 *>(tb + off);
                    s[i] = *reinterpret_cast<const uint32_t *>(sp + (kk >> 2) * kGroupBytes);
                }
            }
#pragma unroll
            for (int i = 0; i < kDownPF; ++i) {
                const int kk = kb + i;
                if (kk < u1) {
                    const int blk = 4 * kk + q;
                    float p;
                    if (HF32)
                        p = fp4x32_dot_f32(c[i], reinterpret_cast<const float4 *>(smem) +
                                                     ((size_t)j * kp + blk * 32) / 4);
                    else
                        p = fp4x32_dot_bf16(c[i], reinterpret_cast<const uint4 *>(smem) +
                                                      ((size_t)j * kp + blk * 32) / 8);
                    acc = fmaf(p, e8m0_f32((s[i] >> (8 * (kk & 3))) & 255u), acc);
                }
            }
        }
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    // per slot: 16 postscales, then its routing weight (NaN marks a bad id)
    float *pss = red + a.topk * a.S * 16;
    if (lane < 16) red[wave * 16 + lane] = acc;
    if (part == 0 && lane < 16) pss[j * 17 + lane] = psj;
    if (part == 0 && lane == 16) pss[j * 17 + 16] = valid ? wj : __builtin_nanf("");
    __syncthreads();
    if (wave != 0 || lane >= 16) return;
    const int row = tile * 16 + lane;
    float y = 0.0f;
    for (int jj = 0; jj < a.topk; ++jj) {
        float dot = red[(jj * a.S) * 16 + lane];
        for (int pp = 1; pp < a.S; ++pp) dot += red[(jj * a.S + pp) * 16 + lane];
        y += pss[jj * 17 + 16] * (pss[jj * 17 + lane] * dot);
    }
    if (row < a.hidden) store_out(a.y, (int64_t)b * a.hidden + row, y, a.y_bf16);
}

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
                          static_cast<hipStream_t>(stream), ra);
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
    // K-split per slot: up to 16 waves per workgroup in total
    int S = 16 / (int)topk;
    while (S > 1 && (int)ceil_div(g.units, S) < 4) S /= 2;
    a.S = S < 1 ? 1 : S;
    const size_t esz = h_dtype == TT_F32 ? 4 : 2;
    const size_t lds = (size_t)topk * g.units * 128 * esz + (size_t)topk * a.S * 64 +
                       (size_t)topk * 17 * 4;
    if (lds > 64 * 1024) {
        static bool raised[2][64] = {{false}};
        int dev = 0;
        (void)hipGetDevice(&dev);
        const int which = h_dtype == TT_F32;
        if (dev >= 0 && dev < 64 && !raised[which][dev]) {
            const void *fn = which ? reinterpret_cast<const void *>(k_down_combine<true>)
                                   : reinterpret_cast<const void *>(k_down_combine<false>);
            if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) !=
                hipSuccess)
                return fail(TT_E_HIP, "cannot raise the LDS limit of the down kernel");
            raised[which][dev] = true;
        }
        if (lds > 160 * 1024)
            return fail(TT_E_SHAPE, "topk * inter = %lld activations do not fit in LDS",
                        (long long)(topk * inter));
    }
    dim3 grid((unsigned)ceil_div(hidden, kTileRows), (unsigned)batch);
    dim3 block((unsigned)(64 * topk * a.S));
    hipStream_t s = static_cast<hipStream_t>(stream);
    tt_status st =
        h_dtype == TT_F32
            ? launch("moe down + combine", k_down_combine<true>, grid, block, lds, s, a)
            : launch("moe down + combine", k_down_combine<false>, grid, block, lds, s, a);
    if (st == TT_OK) clear_error();
    return st;
}
