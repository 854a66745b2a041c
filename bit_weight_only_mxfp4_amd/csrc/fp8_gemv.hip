// fp8_gemv.hip -- row-scaled FP8 E4M3 matvec (kerbin.cskartikey.dev/
// @satvikhardat, "Dev Log #3 -- SmolLM3-3B Results": the quality FP8 profile
// runs gate/up and the middle down projections as scaled matvecs, the row's
// fp32 sum of weight * activation times the row scale):
//   y[b][r] = scale[r] * sum_k w[r][k] * x[b][k]
// Here it is the dense down projection after the gate/up SwiGLU, so x is that
// call's output h (fp32, or bf16).
//
// Layout (layout.h): 8-row tiles, 1 KiB units of 8 rows x 128 k; lane l of a
// wave loads 16 codes of row l % 8 at k = 128 u + 16 (l / 8).  A down
// projection has few rows and a long K, so 8-row tiles give one workgroup per
// CU on a SmolLM3-shaped down projection (2048 rows -> 256 tiles) where
// 16-row tiles would leave half the chip idle.
//
// One workgroup per tile and NT tokens; wave p owns units [p UPW, p UPW +
// UPW).  Issue order per wave: the activations its units read (straight-line
// buffer loads, zeros past k and past the batch), then its UPW code units,
// then -- in wave 0 -- the tile's row scales.  The activations go to the
// wave's own part of LDS as they are (no barrier: no other wave reads them);
// each unit is consumed as its load lands.  fp32 activations: v_cvt_scalef32_pk_f32_fp8 (scale 1) turns two
// E4M3 codes into two exact fp32 values, one FMA per element accumulates.
// Then xor-shuffles over the 8 pieces of each row.  bf16 activations:
// v_cvt_scalef32_pk_bf16_fp8 turns two codes into two exact bf16 values and
// the bf16 matrix cores take the products (the 8-row tile's even and odd
// pieces as the two halves of the 16 columns, the tokens' matching pieces as
// the rows), leaving one lane exchange per row.  A fixed-order cross-wave sum
// in LDS follows; the row scale multiplies the full sum.
#include "device.h"
#include "tt_internal.h"

namespace tt {

struct F8Args {
    const uint8_t *w;
    int64_t tile_stride;
    int32_t n, k, units, scale_off, ntiles;
    const void *x;      // [batch][k], fp32 or bf16
    int32_t batch;
    void *y;            // [batch][n]
    int32_t y_bf16;
    int32_t ks;         // waves per tile
};

constexpr int kF8Oob = 0x7FFFFF00;  // buffer offset past every range: loads return 0

// 16-byte buffer load under cache policy POLICY (kStreamPolicy for weights)
template <int POLICY>
__device__ __forceinline__ uint4 f8_load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void f8_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// sum_{i<4} E4M3(byte i of c) * x[i], continuing acc
__device__ __forceinline__ float f8x4_dot(uint32_t c, float4 x, float acc) {
    const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
    const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, true);
    acc = fmaf(lo.x, x.x, acc);
    acc = fmaf(lo.y, x.y, acc);
    acc = fmaf(hi.x, x.z, acc);
    return fmaf(hi.y, x.w, acc);
}

// Four E4M3 codes (bytes in k order) -> four exact bf16 values, k order kept.
__device__ __forceinline__ uint2 f8x4_to_bf16x4(uint32_t c) {
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true)));
}

// The argument struct with the leading kernel parameters written in (they
// are preloaded into scalar registers): everything read before the weight
// loads (the tile geometry follows from k), and the output, which the tail
// after the last barrier needs (read from argument memory there, it would
// add a memory round trip to the end of every call).
__device__ __forceinline__ F8Args f8_hot_args(F8Args a, const uint8_t *w, const void *x,
                                              int32_t k, int32_t batch, int32_t ks, int32_t n,
                                              void *y, int32_t y_bf16) {
    const F8Geom g = f8_geom(k);
    a.w = w;
    a.x = x;
    a.k = k;
    a.units = (int32_t)g.units;
    a.scale_off = (int32_t)g.scale_off;
    a.tile_stride = g.stride;
    a.batch = batch;
    a.ks = ks;
    a.n = n;
    a.y = y;
    a.y_bf16 = y_bf16;
    return a;
}

template <int UPW, int NT, bool XF32>
__global__ __launch_bounds__(1024) void k_fp8_gemv(const uint8_t *w, const void *x, int32_t k,
                                                   int32_t batch, int32_t ks_, int32_t rows,
                                                   void *y, int32_t y_bf16, F8Args cold) {
    const F8Args a = f8_hot_args(cold, w, x, k, batch, ks_, rows, y, y_bf16);
    extern __shared__ __align__(16) uint8_t smem[];
    const int ks = a.ks;
    constexpr int XSZ = XF32 ? 4 : 2;            // staged bytes per activation
    const int kp = ks * UPW * kF8UnitK;           // staged K per token, zero past k
    float *xs = reinterpret_cast<float *>(smem);  // [NT][kp] fp32, or bf16 as uint16
    float *red = reinterpret_cast<float *>(smem + (size_t)NT * kp * XSZ);  // [ks][NT][8]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = blockIdx.x, t0 = blockIdx.y * NT;
    const int nt = min(NT, a.batch - t0);

    // 1. activations of the wave's own units: 16-byte chunks of 4 fp32 or 8
    //    bf16 elements, chunk j * 64 + lane of the wave's slice per token
    constexpr int EPC = XF32 ? 4 : 8;
    constexpr int XL = XF32 ? UPW / 2 : UPW / 4;  // chunks per lane per token
    constexpr int XC = NT * XL;
    const int u0 = wave * UPW;
    const int cw0 = u0 * kF8UnitK / EPC;  // first chunk of the wave's slice
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.x), 0, a.batch * a.k * (XF32 ? 4 : 2), 0x00020000);
    uint4 xv[XC];
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const int t = c / XL, e0 = (cw0 + (c % XL) * 64 + lane) * EPC;
        const bool ok = t < nt && e0 < a.k;
        xv[c] = f8_load16<0>(xr, ok ? ((t0 + t) * a.k + e0) * (XF32 ? 4 : 2) : kF8Oob);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. weights, then the row scales for the wave that finishes the tile
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.w + (int64_t)tile * a.tile_stride), 0, (int)a.tile_stride,
        0x00020000);
    uint4 cu[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i)
        cu[i] = f8_load16<kStreamPolicy>(rs, u0 + i < a.units ? (u0 + i) * kUnitBytes + lane * 16 : kF8Oob);
    const float scale = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(
                   rs, (wave == 0 && lane < kF8TileRows) ? a.scale_off + lane * 4 : kF8Oob, 0,
                   kStreamPolicy));

    // 3. the slice to LDS as it is (fp32 or bf16); only this wave reads it
    //    back, and a wave's LDS accesses complete in order: no barrier
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const int t = c / XL;
        reinterpret_cast<uint4 *>(xs)[t * (kp / EPC) + cw0 + (c % XL) * 64 + lane] = xv[c];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

    // 4. consume the units in load order: lane (r, q) covers k = 128 u + 16 q
    const int q = lane >> 3;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    if constexpr (XF32) {
        if constexpr (NT == 1) {
            // unit i + 1's activations are read from LDS while unit i is
            // summed (one token: the registers for it are free)
            float4 xcur[NT][4], xnext[NT][4];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float4 *xg =
                    reinterpret_cast<const float4 *>(xs + t * kp + kF8UnitK * u0 + 16 * q);
#pragma unroll
                for (int j = 0; j < 4; ++j) xcur[t][j] = xg[j];
            }
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                if (i + 1 < UPW) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const float4 *xg = reinterpret_cast<const float4 *>(
                            xs + t * kp + kF8UnitK * (u0 + i + 1) + 16 * q);
#pragma unroll
                        for (int j = 0; j < 4; ++j) xnext[t][j] = xg[j];
                    }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    float d0 = f8x4_dot(cu[i].x, xcur[t][0], 0.0f);
                    float d1 = f8x4_dot(cu[i].y, xcur[t][1], 0.0f);
                    d0 = f8x4_dot(cu[i].z, xcur[t][2], d0);
                    d1 = f8x4_dot(cu[i].w, xcur[t][3], d1);
                    acc[t] += d0 + d1;
                }
                if (i + 1 < UPW) {
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int j = 0; j < 4; ++j) xcur[t][j] = xnext[t][j];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float4 *xg = reinterpret_cast<const float4 *>(xs + t * kp +
                                                                        kF8UnitK * (u0 + i) + 16 * q);
                    float d0 = f8x4_dot(cu[i].x, xg[0], 0.0f);
                    float d1 = f8x4_dot(cu[i].y, xg[1], 0.0f);
                    d0 = f8x4_dot(cu[i].z, xg[2], d0);
                    d1 = f8x4_dot(cu[i].w, xg[3], d1);
                    acc[t] += d0 + d1;
                }
            }
        }
        // the 8 pieces of each row -> row partial in lanes r (0..7)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = sum_xor32(sum_xor16(sum_xor8(acc[t])));
    } else {
        // bf16 activations on the matrix cores (v_mfma_f32_16x16x32_bf16,
        // two per unit: elements 0..7 and 8..15 of the lane's piece).  B =
        // the lane's codes as exact bf16: column c = lane % 16 is tile row
        // c % 8 with the pieces of parity c / 8, k block = lane / 16, so the
        // lane's own piece 2 (lane / 16) + (lane / 8) % 2 sits where it was
        // loaded.  A row i carries token i % 8's activations of the pieces of
        // parity i / 8 (rows past the batch repeat the last token; their
        // outputs are never used).  Rows t, columns r (< 8) then hold the
        // even pieces' sum of tile row r for token t, rows 8 + t, columns
        // 8 + r the odd pieces' sum: lanes r and r + 40, element t.
        const int ri = lane & 15, kb = lane >> 4;
        const int ta = min(ri & 7, NT - 1), par = ri >> 3;
        static_assert(NT <= 4, "tokens of a pass fit one C element each");
        const uint16_t *xa0 =
            reinterpret_cast<const uint16_t *>(xs) + ta * kp + 16 * (2 * kb + par);
        f32x4_t c0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            const uint4 *xg = reinterpret_cast<const uint4 *>(xa0 + kF8UnitK * (u0 + i));
            const uint4 xlo = xg[0], xhi = xg[1];
            const uint2 e0 = f8x4_to_bf16x4(cu[i].x), e1 = f8x4_to_bf16x4(cu[i].y);
            const uint2 e2 = f8x4_to_bf16x4(cu[i].z), e3 = f8x4_to_bf16x4(cu[i].w);
            const uint4 w0 = make_uint4(e0.x, e0.y, e1.x, e1.y);
            const uint4 w1 = make_uint4(e2.x, e2.y, e3.x, e3.y);
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, xlo), __builtin_bit_cast(bf16x8_t, w0), c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, xhi), __builtin_bit_cast(bf16x8_t, w1), c1, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float v = c0[t] + c1[t];
            acc[t] = v + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                       (lane + 40) * 4, __builtin_bit_cast(int, v)));
        }
    }
    if (ks > 1) {
        if (lane < kF8TileRows)
#pragma unroll
            for (int t = 0; t < NT; ++t) red[(wave * NT + t) * kF8TileRows + lane] = acc[t];
        f8_lds_barrier();
        if (wave != 0) return;
        if (lane < kF8TileRows)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float v = red[t * kF8TileRows + lane];
                for (int w = 1; w < ks; ++w) v += red[(w * NT + t) * kF8TileRows + lane];
                acc[t] = v;
            }
    }
    const int row = tile * kF8TileRows + lane;
    if (lane < kF8TileRows && row < a.n)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < nt) store_out(a.y, (int64_t)(t0 + t) * a.n + row, scale * acc[t], a.y_bf16);
}

namespace {

constexpr size_t kF8LdsMax = 160 * 1024;

size_t f8_lds(int ks, int upw, int nt, bool xf32) {
    return (size_t)nt * ks * upw * kF8UnitK * (xf32 ? 4 : 2) + (size_t)ks * nt * kF8TileRows * 4;
}

template <int UPW, int NT, bool XF32>
tt_status launch_f8(F8Args a, hipStream_t s) {
    a.ks = (int32_t)ceil_div(a.units, UPW);
    const size_t lds = f8_lds(a.ks, UPW, NT, XF32);
    auto kern = k_fp8_gemv<UPW, NT, XF32>;
    if (lds > 64 * 1024) TT_TRY((raise_lds_limit<k_fp8_gemv<UPW, NT, XF32>>("fp8 gemv")));
    dim3 grid((unsigned)a.ntiles, (unsigned)ceil_div(a.batch, NT));
    return launch("fp8 gemv", kern, grid, dim3(64 * a.ks), lds, s, a.w, a.x, a.k, a.batch, a.ks,
                  a.n, a.y, a.y_bf16, a);
}

// registers a wave holds for loads in flight: its code units plus NT tokens'
// activation chunks (kept within 24 x 4 VGPRs at 16 waves per workgroup)
constexpr bool f8_fits(int upw, int nt, bool xf32) {
    return upw + nt * (xf32 ? upw / 2 : upw / 4) <= 24;
}

template <int UPW, bool XF32>
tt_status launch_f8_nt(const F8Args &a, hipStream_t s) {
    // tokens per weight pass: as many as the batch needs, as LDS and
    // registers allow
    const int ks = (int)ceil_div(a.units, UPW);
    int nt = a.batch == 1 ? 1 : a.batch == 2 ? 2 : 4;
    while (nt > 1 && (f8_lds(ks, UPW, nt, XF32) > kF8LdsMax || !f8_fits(UPW, nt, XF32))) nt /= 2;
    if constexpr (f8_fits(UPW, 4, XF32))
        if (nt == 4) return launch_f8<UPW, 4, XF32>(a, s);
    if constexpr (f8_fits(UPW, 2, XF32))
        if (nt == 2) return launch_f8<UPW, 2, XF32>(a, s);
    return launch_f8<UPW, 1, XF32>(a, s);
}

template <bool XF32>
tt_status launch_f8_upw(const F8Args &a, hipStream_t s) {
    // units per wave: the smallest that keeps a tile within 16 waves
    if (ceil_div(a.units, 4) <= 16) return launch_f8_nt<4, XF32>(a, s);
    if (ceil_div(a.units, 8) <= 16) return launch_f8_nt<8, XF32>(a, s);
    if (ceil_div(a.units, 12) <= 16) return launch_f8_nt<12, XF32>(a, s);
    return launch_f8_nt<16, XF32>(a, s);
}

}  // namespace
}  // namespace tt

using namespace tt;

extern "C" tt_status tt_fp8_gemv(const void *w_packed, int64_t n, int64_t k, const void *x,
                                 int32_t x_dtype, int64_t batch, void *y, int32_t y_dtype,
                                 void *stream) {
    TT_TRY(check_ptr(w_packed, "w_packed"));
    TT_TRY(check_ptr(x, "x"));
    TT_TRY(check_ptr(y, "y"));
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, "n"));
    TT_TRY(check_range(k, 1, TT_MAX_K_FP8, "k"));
    TT_TRY(check_range(batch, 1, TT_MAX_BATCH, "batch"));
    TT_TRY(check_dtype(x_dtype, "x_dtype"));
    TT_TRY(check_dtype(y_dtype, "y_dtype"));
    const bool xf32 = x_dtype == TT_F32;
    if (k % (xf32 ? 4 : 8))
        return fail(TT_E_SHAPE, "k = %lld is not a multiple of %d (%s activations)",
                    (long long)k, xf32 ? 4 : 8, xf32 ? "fp32" : "bf16");
    TT_TRY(check_align(w_packed, 16, "w_packed"));
    TT_TRY(check_align(x, 16, "x"));
    TT_TRY(check_align(y, y_dtype == TT_F32 ? 4 : 2, "y"));
    const F8Geom g = f8_geom(k);
    F8Args a;
    a.w = static_cast<const uint8_t *>(w_packed);
    a.tile_stride = g.stride;
    a.n = (int32_t)n;
    a.k = (int32_t)k;
    a.units = (int32_t)g.units;
    a.scale_off = (int32_t)g.scale_off;
    a.ntiles = (int32_t)ceil_div(n, kF8TileRows);
    a.x = x;
    a.batch = (int32_t)batch;
    a.y = y;
    a.y_bf16 = y_dtype == TT_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tt_status st = xf32 ? launch_f8_upw<true>(a, s) : launch_f8_upw<false>(a, s);
    if (st == TT_OK) clear_error();
    return st;
}
