// mxfp4_gateup.hip -- MXFP4 gate/up projection fused with the row postscale
// and SwiGLU, dense and routed-expert, for gfx950.
//
// What is computed ("Dev Log #4", section "Where Blackwell helps": 4-bit
// codes under block scales against bf16 activations, the row postscale on the
// finished sum; "Dev Log #2": gated activation; stardance page, "numerical
// drift & speedups": the same over the selected experts):
//   out[r] = silu(ps_g[r] * (Wg x)[r]) * (ps_u[r] * (Wu x)[r]).
//
// Batch 1 and 2 (and the routed experts, one token per slot) run on the
// gfx950 scaled matrix instruction: the packed FP4 tile units and their E8M0
// block scales go to v_mfma_scale_f32_16x16x128_f8f6f4 as they are loaded,
// against the bf16 activations split into two E4M3 parts with E8M0 scales.
// One workgroup per 1-2 tiles of 16 rows (8 gate + 8 up rows of the same
// output features), ks waves splitting the tile's K units; a fixed-order
// cross-wave sum gives the row dot products, and the postscale and SwiGLU
// run in registers.
//
// Batch 3..32 runs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16): the same
// 16-byte loads become bf16 A operands with the block scale folded into the
// conversion, and each wave keeps the activations of up to 32 tokens over its
// slice of K in registers as B operands while it streams a run of tiles.
#include <algorithm>

#include "device.h"
#include "tt_internal.h"

namespace tt {

struct GateUpArgs {
    const uint8_t *w;       // gate/up pack, or the bank base for experts
    int64_t expert_stride;  // bytes per expert pack
    int64_t tile_stride;
    int32_t ntiles;         // tiles per pack
    int32_t nb, units, qv_last;
    int32_t scale_off, ps_off;
    const uint16_t *x;      // [tokens][hidden] bf16
    int32_t hidden;
    const int32_t *ids;     // [slots] expert ids, or NULL for the dense call
    int32_t topk, n_experts;
    void *out;              // [slots][inter]
    int32_t out_bf16;
    int32_t inter;
    int32_t batch;          // tokens (dense calls)
    int32_t ks;             // waves per tile (scaled-MFMA path: the K split)
    const uint16_t *logits; // fused routing: bf16 [tokens][n_experts], or NULL
    int32_t *ids_out;       // fused routing: chosen experts [slots]
    float *w_out;           // fused routing: routing weights [slots]
};

// The argument struct with the leading kernel parameters of the scaled-MFMA
// kernel written in: every field that kernel reads before its weight loads
// comes from those parameters (preloaded), in dense and routed calls alike.
// The tile geometry follows from the block count nb (K = 32 nb); the expert
// stride of a bank is ntiles whole tiles; rt = topk | n_experts << 16 for
// routed calls.
__device__ __forceinline__ GateUpArgs gu_hot_args(GateUpArgs a, const uint8_t *w,
                                                  const uint16_t *x, const int32_t *ids,
                                                  const uint16_t *logits, int32_t nb,
                                                  int32_t ntiles, int32_t ks, int32_t batch,
                                                  int32_t rt) {
    const MxGeom g = mx_geom(32 * (int64_t)nb);
    a.w = w;
    a.x = x;
    a.ids = ids;
    a.logits = logits;
    a.nb = nb;
    a.units = (int32_t)g.units;
    a.qv_last = (int32_t)g.qv_last;
    a.scale_off = (int32_t)g.scale_off;
    a.ps_off = (int32_t)g.ps_off;
    a.tile_stride = g.stride;
    a.hidden = 32 * nb;
    a.ntiles = ntiles;
    a.ks = ks;
    a.batch = batch;
    a.topk = rt & 0xFFFF;
    a.n_experts = rt >> 16;
    a.expert_stride = (int64_t)ntiles * g.stride;
    return a;
}

// Orderable key of (bf16 logit, expert index): larger logit first, then the
// lower index; -0 folds onto +0 (the same ranking rule as the routing call).
__device__ __forceinline__ uint32_t gu_route_key(uint32_t bits, int e) {
    bits = (bits == 0x8000u) ? 0u : bits;
    const uint32_t ord = (bits & 0x8000u) ? (~bits & 0xFFFFu) : (bits | 0x8000u);
    return (ord << 16) | (0xFFFFu - (uint32_t)e);
}

// Maximum over the wave: DPP steps within each row of 16 lanes (quad swaps,
// then the half-row and row mirrors), then the four row maxima read out as
// scalars.  No LDS permutes.
__device__ __forceinline__ uint32_t gu_wave_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Expert of slot j for one token, by iterated wave maxima over the keys of
// the token's logits (4 per lane; keys past the expert count are 0, below
// every real key).  A key carries both its logit and its expert index, so
// rank r's logit and expert come straight out of the r-th maximum.  With
// want_w the routing weight follows: the softmax of the topk selected logits,
// summed in rank order.  No LDS and no barrier: every wave does this itself.
__device__ __forceinline__ int gu_route_topj(uint32_t key[4], int topk, int j, bool want_w,
                                             float *wj) {
    const int need = want_w ? topk : j + 1;
    float sel[TT_MAX_TOPK], selj = 0.0f;
    int e = 0;
#pragma unroll
    for (int r = 0; r < TT_MAX_TOPK; ++r) {
        sel[r] = 0.0f;
        if (r < need) {
            const uint32_t m = gu_wave_max(max(max(key[0], key[1]), max(key[2], key[3])));
            const uint32_t ord = m >> 16;
            const uint32_t bits = (ord & 0x8000u) ? (ord & 0x7FFFu) : (~ord & 0xFFFFu);
            sel[r] = bf16_bits_to_f32(bits);
            if (r == j) {
                e = (int)(0xFFFFu - (m & 0xFFFFu));
                selj = sel[r];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) key[i] = key[i] == m ? 0u : key[i];
        }
    }
    if (want_w) {
        float den = 0.0f;
#pragma unroll
        for (int r = 0; r < TT_MAX_TOPK; ++r)
            if (r < topk) den += expf(sel[r] - sel[0]);
        *wj = expf(selj - sel[0]) / den;
    }
    return e;
}

// Tuning of the scaled-MFMA path: units of K per wave (4 or 8) and tiles per
// workgroup.
#ifndef TT_GATEUP_UPW
#define TT_GATEUP_UPW 4
#endif
#ifndef TT_GATEUP_TPB
#define TT_GATEUP_TPB 2
#endif
// Largest dense batch on the scaled-MFMA path (2 tokens per workgroup).
#ifndef TT_GATEUP_MX_MAXB
#define TT_GATEUP_MX_MAXB 2
#endif
constexpr size_t kMaxLdsBytes = 160 * 1024;
constexpr int kMaxWavesPerTile = 16;
constexpr int kOob = 0x7FFFFF00; // buffer offset past every tile: loads return 0

// Byte offset of lane `lane`'s 16 code bytes in unit kk.  Lanes whose piece
// lies past the row end (only in the last unit) re-read piece 0 of their row;
// their activations are zero in LDS and their scale byte is 127, so they add
// exactly zero.
__device__ __forceinline__ int code_off(int kk, int lane, int units, int qv_last) {
    return kk * kUnitBytes +
           ((kk == units - 1 && (lane >> 4) >= qv_last) ? (lane & 15) * 16 : lane * 16);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int64_t bytes) {
    // raw buffer: stride 0, loads at offsets >= bytes return zero
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// LDS-only workgroup barrier: orders LDS traffic without waiting for the
// weight loads still in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders one wave's own LDS writes before its later LDS reads, with no
// workgroup barrier.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Scaled-MFMA path (batch 1 and 2 and the routed slots): each packed unit
// and its E8M0 scale byte go to v_mfma_scale_f32_16x16x128_f8f6f4 as loaded
// (layouts and the two-part E4M3 activations: device.h).  Token t's hi part
// is B column t and its lo part column 8 + t; column 8 + t is added onto
// column t after the last unit.
template <int NTOK>
struct MxLds {
    int kp;  // staged elements per token (a multiple of 512)
    __device__ int q_bytes() const { return NTOK * 2 * kp; }
    __device__ int s_bytes() const { return NTOK * 2 * (kp / 32); }
    // E4M3 part hl (0 hi, 1 lo) of token t
    __device__ int q_off(int t, int hl) const { return (t * 2 + hl) * kp; }
    // E8M0 byte of part hl of token t, group g (block 4u + g) of unit u
    __device__ int s_off(int t, int hl, int g, int u) const {
        return q_bytes() + ((t * 2 + hl) * 4 + g) * (kp / 128) + u;
    }
    __device__ int zero_off() const { return q_bytes() + s_bytes(); }   // 32 zero bytes
    __device__ int red_off() const { return zero_off() + 32; }          // [waves][NTOK][16] f32
};

template <int NTOK>
__host__ __device__ constexpr size_t mx_lds_bytes(int ks, int upw, int tpb) {
    return (size_t)NTOK * 2 * ks * upw * 128 + (size_t)NTOK * 2 * ks * upw * 4 + 32 +
           (size_t)tpb * ks * NTOK * 64;
}

// Workgroup = TPB tiles x ks waves, wave (t, p) owns units [p UPW, p UPW +
// UPW) of tile blockIdx.x * TPB + t.  NTOK tokens per workgroup (dense
// calls: tokens blockIdx.y * NTOK ..; routed calls: NTOK = 1, slot
// blockIdx.y).  Issue order per wave: its share of the activations, then
// each scale dword followed by its four units, then the postscales; the
// activations are split into their E4M3 parts into LDS, and after an
// LDS-only barrier each unit goes to the matrix core as its load lands.
// Lanes whose piece of the last unit lies past the row end read whatever
// follows (FP4 codes have no NaN; the pack gives them scale byte 127) against
// zero activations, so they add exactly zero; loads past the tile return 0.
template <int UPW, int TPB, int NTOK>
__global__ __launch_bounds__(1024) void k_gateup_mx(const uint8_t *w, const uint16_t *x,
                                                    const int32_t *ids, const uint16_t *logits,
                                                    int32_t nb, int32_t ntiles, int32_t ks_,
                                                    int32_t batch, int32_t rt, GateUpArgs cold) {
    static_assert(UPW % 4 == 0 && UPW <= 16, "units per wave");
    const GateUpArgs a = gu_hot_args(cold, w, x, ids, logits, nb, ntiles, ks_, batch, rt);
    static_assert(NTOK == 1 || NTOK == 2 || NTOK == 4 || NTOK == 8, "tokens per workgroup");
    extern __shared__ __align__(16) uint8_t smem[];
    const int ks = a.ks;
    const MxLds<NTOK> L{ks * UPW * 128};
    const int tid = threadIdx.x, lane = tid & 63;
    const int nthreads = 64 * TPB * a.ks;  // the launch's block size
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tsub = wave / ks, part = wave - tsub * ks;
    const int tile = blockIdx.x * TPB + tsub, slot = blockIdx.y;
    const bool routed = a.ids || a.logits;
    const int tok0 = routed ? slot / a.topk : slot * NTOK;   // first token of the workgroup
    const int ntok = routed ? 1 : min(NTOK, a.batch - tok0);

    // 1. activations: 16-byte chunks (zero past K and past the batch);
    //    chunk i of a token is elements 8i .. 8i+7.  One-tile workgroups:
    //    each wave fetches only the UPW * 16 chunks per token that its own
    //    units read (chunk part * UPW * 16 + 64 c + lane), and stages them in
    //    its own part of LDS.  Otherwise the tiles of the workgroup share
    //    one staging of all NTOK * kp / 8 chunks behind a barrier.
    constexpr bool kOwnX = TPB == 1;
    constexpr int XC = NTOK * UPW / 4;   // >= chunks per thread (nthreads >= 64 ks)
    const int tchunks = L.kp / 8, xvalid = a.hidden / 8;
    const auto xchunk = [&](int j, int &t, int &ci) {
        if (kOwnX) {
            t = j / (UPW / 4);
            ci = part * UPW * 16 + (j % (UPW / 4)) * 64 + lane;
        } else {
            const int idx = tid + j * nthreads;
            t = idx / tchunks;
            ci = idx - t * tchunks;
        }
    };
    uint4 xv[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
        int t, ci;
        xchunk(j, t, ci);
        xv[j] = (t < ntok && ci < xvalid)
                    ? reinterpret_cast<const uint4 *>(a.x + (int64_t)(tok0 + t) * a.hidden)[ci]
                    : make_uint4(0, 0, 0, 0);
    }

    const uint8_t *base = a.w;
    int route_e = 0;
    float route_w = 0.0f;
    if (a.logits) {
        const uint16_t *lb = a.logits + (int64_t)tok0 * a.n_experts;
        uint32_t key[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ei = lane + 64 * i;
            key[i] = 0u;
            if (64 * i < a.n_experts) {  // uniform
                const uint32_t raw = lb[min(ei, a.n_experts - 1)];
                key[i] = ei < a.n_experts ? gu_route_key(raw, ei) : 0u;
            }
        }
        float wj = 0.0f;
        const int j = slot - tok0 * a.topk;
        const bool writer = blockIdx.x == 0;
        const int e = gu_route_topj(key, a.topk, j, writer, &wj);
        route_e = e;
        route_w = wj;
        base += (int64_t)e * a.expert_stride;
    } else if (a.ids) {
        const int e = a.ids[slot];
        if (e < 0 || e >= a.n_experts) {
            for (int i = tid; i < TPB * 8; i += nthreads) {
                const int pair = blockIdx.x * TPB * 8 + i;
                if (pair < a.inter)
                    store_out(a.out, (int64_t)slot * a.inter + pair, __builtin_nanf(""),
                              a.out_bf16);
            }
            return;
        }
        base += (int64_t)e * a.expert_stride;
    }

    // 2. weights
    const bool tile_ok = tile < a.ntiles;
    const uint8_t *tb = base + (int64_t)(tile_ok ? tile : 0) * a.tile_stride;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(tb, a.tile_stride);
    const int u0 = part * UPW;
    const int n = tile_ok ? max(0, min(UPW, a.units - u0)) : 0;
    uint4 c[UPW];
    uint32_t sd[UPW / 4];
    const int voff = u0 * kUnitBytes + lane * 16;
    const int soff = a.scale_off + (u0 >> 2) * kGroupBytes + lane * 4;
#pragma unroll
    for (int g = 0; g < UPW / 4; ++g) {
        sd[g] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * g < n ? soff + g * kGroupBytes : kOob,
                                                     0, kStreamPolicy);
#pragma unroll
        for (int i = 4 * g; i < 4 * g + 4; ++i)
            c[i] = load16(rs, i < n ? voff + i * kUnitBytes : kOob);
    }
    // postscales for the finishing lanes (lane 8t + r finishes gate row r
    // and up row r + 8), fetched with the weights by the finishing wave
    // only: lane l loads row l % 16, and a DPP rotate by 8 inside the row of
    // 16 lanes brings the partner row
    const int fr = lane & 7;
    const bool fin = part == 0 && tile_ok;
    float ps_own = 0.0f;
    if (fin)  // uniform
        ps_own = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, a.ps_off + (lane & 15) * 4, 0, kStreamPolicy));
    // the routing outputs (their pointers come with the argument struct)
    if (a.logits && blockIdx.x == 0 && tid == 0) {
        a.ids_out[slot] = route_e;
        a.w_out[slot] = route_w;
    }
    // keep every load above the activation split
    __builtin_amdgcn_sched_barrier(0);

    // 3. activations -> E4M3 parts and their scales in LDS
#pragma unroll
    for (int j = 0; j < XC; ++j) {
        int t, ci;
        xchunk(j, t, ci);
        uint2 hi, lo;
        const uint32_t sh = split_chunk(xv[j], &hi, &lo);
        if (t < NTOK) {
            *reinterpret_cast<uint2 *>(smem + L.q_off(t, 0) + ci * 8) = hi;
            *reinterpret_cast<uint2 *>(smem + L.q_off(t, 1) + ci * 8) = lo;
            if ((ci & 3) == 0) {
                const int blk = ci >> 2;
                smem[L.s_off(t, 0, blk & 3, blk >> 2)] = (uint8_t)sh;
                smem[L.s_off(t, 1, blk & 3, blk >> 2)] = (uint8_t)(sh - 4u);
            }
        }
    }
    if (kOwnX) {
        // every wave writes the same zeros before it reads them; a wave's
        // own LDS accesses complete in order
        if (lane < 8) reinterpret_cast<uint32_t *>(smem + L.zero_off())[lane] = 0u;
        wave_lds_fence();
    } else {
        if (tid < 8) reinterpret_cast<uint32_t *>(smem + L.zero_off())[tid] = 0u;
        lds_barrier();
    }

    // 4. the units in load order, one scaled MFMA each
    const int col = lane & 15, grp = lane >> 4;
    const int ct = col & 7, hl = col >> 3;
    const bool bact = ct < ntok;
    const int qbase = bact ? L.q_off(ct, hl) + u0 * 128 + 16 * grp : L.zero_off();
    const int qstep = bact ? 128 : 0;
    const int sbase = L.s_off(bact ? ct : 0, hl, grp, u0);
    f32x4_t C = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t sb = 0x7F7F7F7Fu;  // columns without a token: scale 1, zero data
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        if ((i & 3) == 0 && bact) sb = *reinterpret_cast<const uint32_t *>(smem + sbase + i);
        const uint4 b0 = *reinterpret_cast<const uint4 *>(smem + qbase + i * qstep);
        const uint4 b1 = *reinterpret_cast<const uint4 *>(smem + qbase + i * qstep + (bact ? 64 : 16));
        const i32x8_t B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                           (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        const i32x8_t A = {(int)c[i].x, (int)c[i].y, (int)c[i].z, (int)c[i].w, 0, 0, 0, 0};
        C = mfma_fp4_fp8(i & 3, A, B, C, sd[i >> 2], sb);
    }

    // 5. lo column 8 + t onto column t (DPP row shift left by 8), the
    //    partial rows to LDS, one barrier, then the fixed-order sum over the
    //    K parts by the tile's first wave: lane 8t + r finishes pair r of
    //    token t (gate row r, up row r + 8)
    const u32x4_t cw = __builtin_bit_cast(u32x4_t, C);
    f32x4_t y;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        y[r] = C[r] + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, (int)cw[r], 0x108,
                                                                            0xF, 0xF, false));
    float *red = reinterpret_cast<float *>(smem + L.red_off());
    if (col < ntok)  // lane (t, g): rows 4g .. 4g+3 of token t
        *reinterpret_cast<f32x4_t *>(red + (wave * NTOK + col) * 16 + 4 * grp) = y;
    lds_barrier();
    const int ft = lane >> 3;
    if (part != 0 || !tile_ok) return;
    const float ps_other = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, ps_own), 0x128, 0xF, 0xF,
                                           false));
    const float psg = (lane & 8) ? ps_other : ps_own;
    const float psu = (lane & 8) ? ps_own : ps_other;
    if (ft >= ntok) return;
    // the K parts' partial rows, four LDS reads in flight at a time
    // (indexes clamped into the table, the surplus masked), summed in order
    float g = 0.0f, u = 0.0f;
    for (int p0 = 0; p0 < ks; p0 += 4) {
        float gv[4], uv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float *rp = red + ((tsub * ks + min(p0 + j, ks - 1)) * NTOK + ft) * 16;
            gv[j] = rp[fr];
            uv[j] = rp[fr + 8];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            g = p0 + j < ks ? g + gv[j] : g;
            u = p0 + j < ks ? u + uv[j] : u;
        }
    }
    const int pair = tile * 8 + fr;
    const int orow = routed ? slot : tok0 + ft;
    if (pair < a.inter)
        store_out(a.out, (int64_t)orow * a.inter + pair, silu(g * psg) * (u * psu), a.out_bf16);
}

// MFMA path (batch 2..32).  NCOL column blocks of 16 tokens.  A workgroup of
// 8 waves owns a contiguous run of at most TMAX tiles; wave p owns K-chunks
// p, p + 8, ... of 2 units (256 elements) each.  For its K-chunk a wave copies
// the activations of all tokens over those 256 elements into a private LDS
// slice (direct buffer-to-LDS loads, one token row of 512 bytes per half
// wave, rotated by the token index so the 16 tokens of a B operand fall on
// different banks), reads its B operands from there once, and keeps them in
// registers while it streams the weights of every tile of the run through
// the matrix cores.  No workgroup barrier precedes the first MFMA.  The 8
// partial tiles are then summed through LDS in a fixed order after one
// barrier; the wave that finishes tile t (t = p) prefetched its postscales.
// With 32 tokens a wave keeps only mfma_ahead() + 1 tiles' weights in
// flight and issues the next tile's as it starts on one: the requests of the
// whole chip then reach memory roughly in tile order, so every wave's first
// tiles land early and its matrix work overlaps the stream instead of
// trailing it.  With one block of 16 tokens the whole run is issued at once,
// which measured faster there.  Up to 8 tokens the runs are of 3 tiles at
// two workgroups per CU, from 9 to 32 tokens of 6 tiles at one per CU (fewer
// workgroups pull fewer copies of the activations through L2).
constexpr int kMfmaWaves = 8;  // waves per workgroup = K-chunk stride
constexpr int kMfmaUpc = 2;    // units per K-chunk

template <int NCOL, int TMAX> constexpr int mfma_ahead() { return NCOL == 2 ? 2 : TMAX; }

// Tile t of a run, K-chunk at unit u0, fetched inside the tile loop (the
// same loads as the loop that fetches the first tiles)
__device__ __forceinline__ void fetch_mfma_tile(const GateUpArgs &a, int t0, int t, int nt, int u0,
                                                int lane, uint4 (&c)[kMfmaUpc], uint32_t &sd) {
    const bool ok = t < nt;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(a.w + (int64_t)(ok ? t0 + t : 0) * a.tile_stride, ok ? a.tile_stride : 0);
    sd = __builtin_amdgcn_raw_buffer_load_b32(rs, a.scale_off + (u0 >> 2) * kGroupBytes + lane * 4,
                                              0, kStreamPolicy);
#pragma unroll
    for (int u = 0; u < kMfmaUpc; ++u)
        c[u] = load16(rs, u0 + u < a.units ? code_off(u0 + u, lane, a.units, a.qv_last) : kOob);
}

template <int NCOL> constexpr int mfma_slice_bytes() { return NCOL * 16 * 512; }

template <int NCOL, int TMAX>
__global__ __launch_bounds__(64 * kMfmaWaves) void k_gateup_mfma(const uint8_t *w,
                                                                  const uint16_t *x, int32_t nb,
                                                                  int32_t ntiles, int32_t batch,
                                                                  int32_t blocks, GateUpArgs cold) {
    static_assert(TMAX * NCOL * 1024 <= mfma_slice_bytes<NCOL>(), "partials fit the slice");
    const GateUpArgs a = gu_hot_args(cold, w, x, nullptr, nullptr, nb, ntiles, 1, batch, 0);
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int p = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint8_t *slice = smem + p * mfma_slice_bytes<NCOL>();
    const int r = lane & 15, q = lane >> 4;
    const int nkc = (a.units + kMfmaUpc - 1) / kMfmaUpc;
    // balanced split of the tiles over the workgroups: at most TMAX each
    const int t0 = (int)((int64_t)blockIdx.x * a.ntiles / blocks);
    const int nt = (int)((int64_t)(blockIdx.x + 1) * a.ntiles / blocks) - t0;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(a.x, (int64_t)a.batch * a.hidden * 2);

    f32x4_t C[TMAX][NCOL];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int cb = 0; cb < NCOL; ++cb) C[t][cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // postscales of rows 4q .. 4q+3 of tile p, which this wave finishes --
    // every finishing wave, also one whose first K-chunk lies past K (a
    // workgroup may own more tiles than the row has K-chunks); issued ahead
    // of the weights, so the epilogue never waits on a load of its own
    f32x4_t ps4 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (p < nt) {  // uniform
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc(a.w + (int64_t)(t0 + p) * a.tile_stride, a.tile_stride);
        ps4 = __builtin_bit_cast(
            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, a.ps_off + 16 * q, 0, kStreamPolicy));
    }

    for (int kc = p; kc < nkc; kc += kMfmaWaves) {  // one round unless K > 2048
        const int u0 = kc * kMfmaUpc;
        // 1. activations of the K-chunk into the slice: instruction i covers
        //    tokens 2i and 2i+1; slot s of token t holds 16-byte piece
        //    (s - t) mod 32; zeros past the batch and past K
        //    (token pairs past the batch are skipped: their slots only feed
        //    output columns that are never stored)
#pragma unroll
        for (int i = 0; i < NCOL * 8; ++i) {
            if (2 * i >= a.batch) break;
            const int t = 2 * i + (lane >> 5), pc = ((lane & 31) - t) & 31;
            const int k = u0 * 128 + 8 * pc;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void *)(slice + i * 1024), 16,
                (t < a.batch && k < a.hidden) ? (t * a.hidden + k) * 2 : kOob, 0, 0, 0);
        }
        // 2. weights of the first kAhead tiles of the run: the units' scale
        //    dword, then the two units; tiles past the run read zeros
        constexpr int kAhead = mfma_ahead<NCOL, TMAX>();
        uint4 c[TMAX][kMfmaUpc];
        uint32_t sd[TMAX];
#pragma unroll
        for (int t = 0; t < kAhead; ++t) {
            const bool ok = t < nt;
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
                a.w + (int64_t)(ok ? t0 + t : 0) * a.tile_stride, ok ? a.tile_stride : 0);
            sd[t] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, a.scale_off + (u0 >> 2) * kGroupBytes + lane * 4, 0, kStreamPolicy);
#pragma unroll
            for (int u = 0; u < kMfmaUpc; ++u)
                c[t][u] = load16(rs, u0 + u < a.units ? code_off(u0 + u, lane, a.units, a.qv_last)
                                                      : kOob);
        }
        // keep every load above this point: the scheduler would otherwise
        // sink the last ones past the first MFMAs and add a round trip
        __builtin_amdgcn_sched_barrier(0);
        // 3. B operands from the slice: lane (r, q) takes token cb*16 + r at
        //    elements (4u + q)*32 + 8j .. +8, i.e. piece (4u + q)*4 + j
        uint4 xb[kMfmaUpc][4][NCOL];
#pragma unroll
        for (int u = 0; u < kMfmaUpc; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int cb = 0; cb < NCOL; ++cb) {
                    const int t = cb * 16 + r, pc = (4 * u + q) * 4 + j;
                    xb[u][j][cb] =
                        *reinterpret_cast<const uint4 *>(slice + t * 512 + ((pc + t) & 31) * 16);
                }
        // 4. tile by tile, each as soon as its loads land; tile t + kAhead is
        //    fetched before tile t is worked on
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if constexpr (kAhead < TMAX) {
                if (t + kAhead < TMAX)
                    fetch_mfma_tile(a, t0, t + kAhead, nt, u0, lane, c[t + kAhead], sd[t + kAhead]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < kMfmaUpc; ++u) {
                const float sc = e8m0_f32((sd[t] >> (8 * ((u0 + u) & 3))) & 255u);
                const uint32_t cw[4] = {c[t][u].x, c[t][u].y, c[t][u].z, c[t][u].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8_t A = fp4x8_to_bf16x8(cw[j], sc);
#pragma unroll
                    for (int cb = 0; cb < NCOL; ++cb)
                        C[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            A, __builtin_bit_cast(bf16x8_t, xb[u][j][cb]), C[t][cb], 0, 0, 0);
                }
            }
        }
    }

    // 5. partial tiles into the wave's own slice (its B operands are in
    //    registers by now), one barrier, fixed-order sum by the finisher
    const int nparts = min(kMfmaWaves, nkc);
    if (p < nparts) {
        f32x4_t *red = reinterpret_cast<f32x4_t *>(slice);
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
#pragma unroll
            for (int cb = 0; cb < NCOL; ++cb)
                if (t < nt) red[(t * NCOL + cb) * 64 + lane] = C[t][cb];
    }
    lds_barrier();
    if (p >= nt) return;
    const int tile = t0 + p;
#pragma unroll
    for (int cb = 0; cb < NCOL; ++cb) {
        // the partial tiles of all K parts read at once (indexes clamped
        // into the slices, the surplus masked off), summed in part order
        const f32x4_t *red = reinterpret_cast<const f32x4_t *>(smem) + (p * NCOL + cb) * 64 + lane;
        constexpr int kStride = mfma_slice_bytes<NCOL>() / 16;
        f32x4_t v[kMfmaWaves];
#pragma unroll
        for (int s = 0; s < kMfmaWaves; ++s) v[s] = red[min(s, nparts - 1) * kStride];
        f32x4_t y = v[0];
#pragma unroll
        for (int s = 1; s < kMfmaWaves; ++s)
            if (s < nparts) y += v[s];
        // lane (token column r, row group q) holds rows 4q..4q+3 of the tile:
        // gate rows in lanes 0..31, the matching up rows 32 lanes on (a
        // half-wave swap brings them over)
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float g = y[i] * ps4[i];
            const uint32_t gb = __builtin_bit_cast(uint32_t, g);
            const f32x2_t sw =
                __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane32_swap(gb, gb, false, false));
            o[i] = silu(g) * sw.y;
        }
        // pairs 4q .. 4q+3 of token cb*16 + r: one vector store when all four
        // lie inside the row and the address is aligned
        const int token = cb * 16 + r, pair0 = tile * 8 + 4 * q;
        if (lane < 32 && token < a.batch) {
            const int64_t at = (int64_t)token * a.inter + pair0;
            if (a.out_bf16) {
                uint16_t *dst = static_cast<uint16_t *>(a.out) + at;
                if (pair0 + 3 < a.inter && (reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
                    *reinterpret_cast<uint2 *>(dst) =
                        make_uint2(f32_to_bf16_bits(o[0]) | (uint32_t)f32_to_bf16_bits(o[1]) << 16,
                                   f32_to_bf16_bits(o[2]) | (uint32_t)f32_to_bf16_bits(o[3]) << 16);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (pair0 + i < a.inter) dst[i] = f32_to_bf16_bits(o[i]);
                }
            } else {
                float *dst = static_cast<float *>(a.out) + at;
                if (pair0 + 3 < a.inter && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (pair0 + i < a.inter) dst[i] = o[i];
                }
            }
        }
    }
}

namespace {

// Compute units of the current device, queried once per device (several
// host threads may race to fill an entry; they store the same value).
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int UPW, int TPB, int NTOK>
tt_status launch_mx(const GateUpArgs &a, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
    if (lds > 64 * 1024)
        TT_TRY((raise_lds_limit<k_gateup_mx<UPW, TPB, NTOK>>("mxfp4 gate/up (scaled MFMA)")));
    return launch("mxfp4 gate/up (scaled MFMA)", k_gateup_mx<UPW, TPB, NTOK>, grid, block, lds,
                  stream, a.w, a.x, a.ids, a.logits, a.nb, a.ntiles, a.ks, a.batch,
                  a.topk | (a.n_experts << 16), a);
}

template <int UPW, int NTOK>
tt_status launch_mx_upw(GateUpArgs a, int slots, int tpb_max, hipStream_t stream) {
    a.ks = (int32_t)ceil_div(a.units, UPW);
    const int tpb = (a.ks * TT_GATEUP_TPB <= 8 && tpb_max >= TT_GATEUP_TPB) ? TT_GATEUP_TPB : 1;
    const size_t lds = mx_lds_bytes<NTOK>(a.ks, UPW, tpb);
    if (lds > kMaxLdsBytes)
        return fail(TT_E_SHAPE, "hidden = %d with %d tokens: the staged activations do not fit "
                    "in LDS", a.hidden, NTOK);
    dim3 grid((unsigned)ceil_div(a.ntiles, tpb), (unsigned)slots);
    if (tpb == 1) return launch_mx<UPW, 1, NTOK>(a, grid, dim3(64 * a.ks), lds, stream);
    return launch_mx<UPW, TT_GATEUP_TPB, NTOK>(a, grid, dim3(64 * tpb * a.ks), lds, stream);
}

// One or two tokens per workgroup (the routed calls take one).  Every
// workgroup splits the activations of all its tokens over the whole K, so
// that work grows with the batch: at 4 tokens the bf16 MFMA path is as fast,
// at 8 it is clearly faster (measured on SmolLM3-sized layers).
template <int UPW>
tt_status launch_mx_ntok(const GateUpArgs &a, int slots, int dense_batch, int tpb_max,
                         hipStream_t stream) {
    if (dense_batch <= 1) return launch_mx_upw<UPW, 1>(a, slots, tpb_max, stream);
    return launch_mx_upw<UPW, 2>(a, (int)ceil_div(dense_batch, 2), tpb_max, stream);
}

// Units per wave: the tuned target, raised until a tile needs at most 16
// waves (K <= 16384 gives at most 128 units, so 8 units per wave always
// suffice).  A grid of 4-unit waves that overflows what the chip holds at
// once (7-8 waves per SIMD at these register counts) but fits it with 8-unit
// waves in one-tile workgroups switches to those: the routed calls, batch x
// topk slots of every tile, would otherwise run a second, partial round.
tt_status launch_scaled(GateUpArgs a, int slots, hipStream_t stream, int dense_batch = 1) {
    int upw = TT_GATEUP_UPW;
    while (ceil_div(a.units, upw) > kMaxWavesPerTile) upw += 4;
    int tpb_max = TT_GATEUP_TPB;
    const int64_t resident = (int64_t)device_cus() * 4 * 7;
    if (upw == 4 && (int64_t)slots * a.ntiles * ceil_div(a.units, 4) > resident &&
        (int64_t)slots * a.ntiles * ceil_div(a.units, 8) <= resident) {
        upw = 8;
        tpb_max = 1;
    }
    switch (upw) {
        case 4: return launch_mx_ntok<4>(a, slots, dense_batch, tpb_max, stream);
        case 8: return launch_mx_ntok<8>(a, slots, dense_batch, tpb_max, stream);
        default: return fail(TT_E_SHAPE, "hidden = %d needs more than 16 waves per tile", a.hidden);
    }
}

constexpr size_t kMaxLds = 160 * 1024;

size_t mfma_lds(int ncol) { return (size_t)kMfmaWaves * ncol * 16 * 512; }

// Runs of at most TMAX tiles per workgroup (a wave's partial tiles fit its
// activation slice), at most per_cu_max workgroups per CU.
template <int NCOL, int TMAX>
tt_status launch_mfma(const GateUpArgs &a, int per_cu_max, hipStream_t stream) {
    const size_t lds = mfma_lds(NCOL);
    if (lds > 64 * 1024)
        TT_TRY((raise_lds_limit<k_gateup_mfma<NCOL, TMAX>>("mxfp4 gate/up (MFMA path)")));
    // as many workgroups as fit the CUs at once, never more than TMAX tiles
    // per workgroup (the split in the kernel is balanced): shorter runs put
    // more waves on each SIMD.  With one workgroup per CU the longest run
    // sets the time, so the tiles go out in runs of that length over as few
    // workgroups as it takes, since each workgroup pulls the activations of
    // all its tokens over the whole K through L2 (128 KB at 32 tokens, K =
    // 2048): 1376 tiles in runs of 6 take 230 workgroups instead of 256.
    const int64_t per_cu = std::min<int64_t>(per_cu_max, (int64_t)(kMaxLds / lds));
    const int64_t slots = per_cu * device_cus();
    int64_t blocks = std::max<int64_t>(std::min<int64_t>(a.ntiles, slots), ceil_div(a.ntiles, TMAX));
    if (per_cu == 1) blocks = ceil_div(a.ntiles, std::min<int64_t>(TMAX, ceil_div(a.ntiles, slots)));
    return launch("mxfp4 gate/up (MFMA path)", k_gateup_mfma<NCOL, TMAX>, dim3((unsigned)blocks),
                  dim3(64 * kMfmaWaves), lds, stream, a.w, a.x, a.nb, a.ntiles, a.batch, blocks, a);
}

GateUpArgs make_args(const void *w, int64_t inter, int64_t hidden, const void *x,
                     void *out, int32_t out_dtype) {
    const MxGeom g = mx_geom(hidden);
    GateUpArgs a;
    a.w = static_cast<const uint8_t *>(w);
    a.expert_stride = ceil_div(inter, kTileRows / 2) * g.stride;
    a.tile_stride = g.stride;
    a.ntiles = (int32_t)ceil_div(inter, kTileRows / 2);
    a.nb = (int32_t)g.nb;
    a.units = (int32_t)g.units;
    a.qv_last = (int32_t)g.qv_last;
    a.scale_off = (int32_t)g.scale_off;
    a.ps_off = (int32_t)g.ps_off;
    a.x = static_cast<const uint16_t *>(x);
    a.hidden = (int32_t)hidden;
    a.ids = nullptr;
    a.topk = 1;
    a.n_experts = 1;
    a.out = out;
    a.out_bf16 = out_dtype == TT_BF16;
    a.inter = (int32_t)inter;
    a.batch = 1;
    a.ks = 1;
    a.logits = nullptr;
    a.ids_out = nullptr;
    a.w_out = nullptr;
    return a;
}

tt_status check_gateup_common(const void *w, int64_t inter, int64_t hidden, const void *x,
                              int64_t batch, void *out, int32_t out_dtype) {
    TT_TRY(check_ptr(w, "w_gu"));
    TT_TRY(check_ptr(x, "x"));
    TT_TRY(check_ptr(out, "out"));
    TT_TRY(check_range(inter, 1, TT_MAX_ROWS, "inter"));
    TT_TRY(check_range(hidden, 32, TT_MAX_K, "hidden"));
    if (hidden % 32) return fail(TT_E_SHAPE, "hidden = %lld is not a multiple of 32", (long long)hidden);
    TT_TRY(check_range(batch, 1, TT_MAX_BATCH, "batch"));
    TT_TRY(check_dtype(out_dtype, "out_dtype"));
    TT_TRY(check_align(w, 16, "w_gu"));
    TT_TRY(check_align(x, 16, "x"));
    TT_TRY(check_align(out, out_dtype == TT_F32 ? 4 : 2, "out"));
    return TT_OK;
}

}  // namespace
}  // namespace tt

using namespace tt;

extern "C" tt_status tt_mxfp4_gateup_swiglu(const void *w_gu, int64_t inter, int64_t hidden,
                                            const void *x, int64_t batch, void *out,
                                            int32_t out_dtype, void *stream) {
    TT_TRY(check_gateup_common(w_gu, inter, hidden, x, batch, out, out_dtype));
    GateUpArgs a = make_args(w_gu, inter, hidden, x, out, out_dtype);
    a.batch = (int32_t)batch;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tt_status st;
    if (batch == 1)
        st = launch_scaled(a, 1, s);
    else if (batch <= TT_GATEUP_MX_MAXB)
        st = launch_scaled(a, 1, s, (int)batch);
    else if (batch <= 8)  // three-tile runs, two workgroups per CU
        st = launch_mfma<1, 3>(a, 2, s);
    else if (batch <= 16)  // six-tile runs, one workgroup per CU
        st = launch_mfma<1, 6>(a, 1, s);
    else
        st = launch_mfma<2, 6>(a, 1, s);
    if (st == TT_OK) clear_error();
    return st;
}

extern "C" tt_status tt_moe_mxfp4_gateup_swiglu(const void *bank, int64_t n_experts,
                                                int64_t inter, int64_t hidden, const void *x,
                                                int64_t batch, const int32_t *ids, int64_t topk,
                                                void *h, int32_t h_dtype, void *stream) {
    TT_TRY(check_gateup_common(bank, inter, hidden, x, batch, h, h_dtype));
    TT_TRY(check_ptr(ids, "ids"));
    TT_TRY(check_align(ids, 4, "ids"));
    TT_TRY(check_range(n_experts, 1, TT_MAX_EXPERTS, "n_experts"));
    TT_TRY(check_range(topk, 1, n_experts < TT_MAX_TOPK ? n_experts : TT_MAX_TOPK, "topk"));
    GateUpArgs a = make_args(bank, inter, hidden, x, h, h_dtype);
    a.ids = ids;
    a.topk = (int32_t)topk;
    a.n_experts = (int32_t)n_experts;
    tt_status st = launch_scaled(a, (int)(batch * topk), static_cast<hipStream_t>(stream));
    if (st == TT_OK) clear_error();
    return st;
}

extern "C" tt_status tt_moe_mxfp4_route_gateup_swiglu(const void *bank, int64_t n_experts,
                                                      int64_t inter, int64_t hidden,
                                                      const void *x, int64_t batch,
                                                      const void *logits, int64_t topk,
                                                      int32_t *ids, float *w, void *h,
                                                      int32_t h_dtype, void *stream) {
    TT_TRY(check_gateup_common(bank, inter, hidden, x, batch, h, h_dtype));
    TT_TRY(check_ptr(logits, "logits"));
    TT_TRY(check_ptr(ids, "ids"));
    TT_TRY(check_ptr(w, "w"));
    TT_TRY(check_align(logits, 2, "logits"));
    TT_TRY(check_align(ids, 4, "ids"));
    TT_TRY(check_align(w, 4, "w"));
    TT_TRY(check_range(n_experts, 1, TT_MAX_EXPERTS, "n_experts"));
    TT_TRY(check_range(topk, 1, n_experts < TT_MAX_TOPK ? n_experts : TT_MAX_TOPK, "topk"));
    GateUpArgs a = make_args(bank, inter, hidden, x, h, h_dtype);
    a.topk = (int32_t)topk;
    a.n_experts = (int32_t)n_experts;
    a.logits = static_cast<const uint16_t *>(logits);
    a.ids_out = ids;
    a.w_out = w;
    tt_status st = launch_scaled(a, (int)(batch * topk), static_cast<hipStream_t>(stream));
    if (st == TT_OK) clear_error();
    return st;
}
