// dequant.hip -- decoded weights of the packed layouts, for bit-exact checks.
// MXFP4 (OCP MX v1.0): w = E2M1(code) * 2^(e-127), rounded once to fp32; the
// FP4 value is converted exactly by the hardware, the scale multiply is the
// single rounding.  INT4: w = s * (q - z) (exact in fp32).
#include "device.h"
#include "tt_internal.h"

namespace tt {

// One wave per (tile, unit).  row_mode 0: tile row r -> output row 16t + r;
// row_mode 1 (gate/up pack): rows 0..7 -> gate row 8t + r, rows 8..15 -> up
// row 8t + r - 8.
struct MxDequantArgs {
    const uint8_t *w;
    int64_t tile_stride;
    int32_t nrows, k, nb, units, qv_last, scale_off, ps_off, row_mode;
    float *out0, *out1, *ps0, *ps1;
};

__global__ __launch_bounds__(64) void k_mx_dequant(MxDequantArgs da) {
    const uint8_t *w = da.w;
    const int64_t tile_stride = da.tile_stride;
    const int nrows = da.nrows, k = da.k, nb = da.nb, units = da.units, qv_last = da.qv_last;
    const int scale_off = da.scale_off, ps_off = da.ps_off, row_mode = da.row_mode;
    float *out0 = da.out0, *out1 = da.out1, *ps0 = da.ps0, *ps1 = da.ps1;
    const int tile = blockIdx.x, kk = blockIdx.y, lane = threadIdx.x;
    const int r = lane & 15, q = lane >> 4;
    const uint8_t *tb = w + (int64_t)tile * tile_stride;
    int row = tile * 16 + r;
    float *out = out0, *ps = ps0;
    if (row_mode == 1) {
        row = tile * 8 + (r & 7);
        out = (r < 8) ? out0 : out1;
        ps = (r < 8) ? ps0 : ps1;
    }
    const bool row_ok = row < nrows;
    if (kk == 0 && q == 0 && row_ok && ps) ps[row] = reinterpret_cast<const float *>(tb + ps_off)[r];
    const int blk = 4 * kk + q;
    if (!row_ok || !out || blk >= nb || (kk == units - 1 && q >= qv_last)) return;
    const uint4 c = *reinterpret_cast<const uint4 *>(tb + kk * kUnitBytes + lane * 16);
    const uint32_t e = tb[scale_off + (kk >> 2) * kGroupBytes + lane * 4 + (kk & 3)];
    const float sc = e8m0_f32(e);
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    float *o = out + (int64_t)row * k + blk * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], 1.0f, 0);
        f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], 1.0f, 1);
        f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], 1.0f, 2);
        f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], 1.0f, 3);
        o[8 * i + 0] = v0.x * sc;
        o[8 * i + 1] = v0.y * sc;
        o[8 * i + 2] = v1.x * sc;
        o[8 * i + 3] = v1.y * sc;
        o[8 * i + 4] = v2.x * sc;
        o[8 * i + 5] = v2.y * sc;
        o[8 * i + 6] = v3.x * sc;
        o[8 * i + 7] = v3.y * sc;
    }
}

struct I4DequantArgs {
    const uint8_t *w;
    int64_t tile_stride;
    int32_t n, k, units, qv_last, sz_off;
    float *out;
};

__global__ __launch_bounds__(64) void k_i4_dequant(I4DequantArgs da) {
    const uint8_t *w = da.w;
    const int64_t tile_stride = da.tile_stride;
    const int n = da.n, k = da.k, units = da.units, qv_last = da.qv_last, sz_off = da.sz_off;
    float *out = da.out;
    const int tile = blockIdx.x, kk = blockIdx.y, lane = threadIdx.x;
    const int r = lane & 15, q = lane >> 4;
    const int row = tile * 16 + r;
    if (row >= n || (kk == units - 1 && q >= qv_last)) return;
    const uint8_t *tb = w + (int64_t)tile * tile_stride;
    const uint4 c = *reinterpret_cast<const uint4 *>(tb + kk * kUnitBytes + lane * 16);
    const uint32_t sz = *reinterpret_cast<const uint32_t *>(
        tb + sz_off + (kk >> 2) * kGroupBytes + r * 16 + (kk & 3) * 4);
    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xFFFFu));
    const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz >> 16));
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    const int k0 = kk * 128 + q * 32;
    for (int j = 0; j < 32; ++j) {
        if (k0 + j >= k) break;
        const float qv = (float)((cw[j >> 3] >> (4 * (j & 7))) & 15u);
        out[(int64_t)row * k + k0 + j] = (qv - z) * s;
    }
}

struct F8DequantArgs {
    const uint8_t *w;
    int64_t tile_stride;
    int32_t n, k, scale_off;
    float *out, *scale_out;
};

// one wave per (8-row tile, 128-k unit): lane l holds 16 codes of row l % 8
__global__ __launch_bounds__(64) void k_f8_dequant(F8DequantArgs da) {
    const int tile = blockIdx.x, u = blockIdx.y, lane = threadIdx.x;
    const int row = tile * kF8TileRows + (lane & 7), k0 = u * kF8UnitK + 16 * (lane >> 3);
    if (row >= da.n) return;
    const uint8_t *tb = da.w + (int64_t)tile * da.tile_stride;
    if (u == 0 && lane < kF8TileRows && da.scale_out)
        da.scale_out[row] = reinterpret_cast<const float *>(tb + da.scale_off)[lane];
    const uint4 c = *reinterpret_cast<const uint4 *>(tb + u * kUnitBytes + lane * 16);
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    for (int d = 0; d < 4; ++d) {
        const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[d], 1.0f, false);
        const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[d], 1.0f, true);
        const float v[4] = {lo.x, lo.y, hi.x, hi.y};
        for (int j = 0; j < 4; ++j)
            if (k0 + 4 * d + j < da.k) da.out[(int64_t)row * da.k + k0 + 4 * d + j] = v[j];
    }
}

}  // namespace tt

using namespace tt;

namespace {

tt_status mx_dequant(const void *packed, int64_t nrows, int64_t ntiles, int64_t k, int row_mode,
                     float *o0, float *o1, float *p0, float *p1, void *stream) {
    const MxGeom g = mx_geom(k);
    dim3 grid((unsigned)ntiles, (unsigned)g.units);
    MxDequantArgs da{static_cast<const uint8_t *>(packed), g.stride, (int32_t)nrows, (int32_t)k,
                     (int32_t)g.nb, (int32_t)g.units, (int32_t)g.qv_last, (int32_t)g.scale_off,
                     (int32_t)g.ps_off, row_mode, o0, o1, p0, p1};
    return launch("mxfp4 dequantize", k_mx_dequant, grid, dim3(64), 0,
                  static_cast<hipStream_t>(stream), da);
}

tt_status check_mx(const void *packed, int64_t n, int64_t k, const char *nname) {
    TT_TRY(check_ptr(packed, "packed"));
    TT_TRY(check_align(packed, 16, "packed"));
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, nname));
    TT_TRY(check_range(k, 32, TT_MAX_K, "k"));
    if (k % 32) return fail(TT_E_SHAPE, "k = %lld is not a multiple of 32", (long long)k);
    return TT_OK;
}

}  // namespace

extern "C" tt_status tt_mxfp4_dequantize(const void *packed, int64_t n, int64_t k, float *w_out,
                                         float *ps_out, void *stream) {
    TT_TRY(check_mx(packed, n, k, "n"));
    TT_TRY(check_ptr(w_out, "w_out"));
    TT_TRY(check_align(w_out, 4, "w_out"));
    tt_status st = mx_dequant(packed, n, ceil_div(n, 16), k, 0, w_out, nullptr, ps_out,
                              nullptr, stream);
    if (st == TT_OK) clear_error();
    return st;
}

extern "C" tt_status tt_mxfp4_gateup_dequantize(const void *packed, int64_t inter,
                                                int64_t hidden, float *g_out, float *u_out,
                                                float *g_ps, float *u_ps, void *stream) {
    TT_TRY(check_mx(packed, inter, hidden, "inter"));
    if (!g_out && !u_out) return fail(TT_E_NULL, "g_out and u_out are both NULL");
    tt_status st = mx_dequant(packed, inter, ceil_div(inter, 8), hidden, 1, g_out, u_out, g_ps,
                              u_ps, stream);
    if (st == TT_OK) clear_error();
    return st;
}

extern "C" tt_status tt_int4_dequantize(const void *packed, int64_t n, int64_t k, int64_t group,
                                        float *w_out, void *stream) {
    TT_TRY(check_ptr(packed, "packed"));
    TT_TRY(check_ptr(w_out, "w_out"));
    TT_TRY(check_align(packed, 16, "packed"));
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, "n"));
    TT_TRY(check_range(k, 2, TT_MAX_K, "k"));
    if (k % 2) return fail(TT_E_SHAPE, "k = %lld is odd", (long long)k);
    if (group != TT_INT4_GROUP)
        return fail(TT_E_SHAPE, "group = %lld; only %d is supported", (long long)group,
                    TT_INT4_GROUP);
    const I4Geom g = i4_geom(k);
    dim3 grid((unsigned)ceil_div(n, 16), (unsigned)g.units);
    I4DequantArgs da{static_cast<const uint8_t *>(packed), g.stride, (int32_t)n, (int32_t)k,
                     (int32_t)g.units, (int32_t)g.qv_last, (int32_t)g.sz_off, w_out};
    tt_status st = launch("int4 dequantize", k_i4_dequant, grid, dim3(64), 0,
                          static_cast<hipStream_t>(stream), da);
    if (st == TT_OK) clear_error();
    return st;
}

extern "C" tt_status tt_fp8_dequantize(const void *packed, int64_t n, int64_t k, float *w_out,
                                       float *scale_out, void *stream) {
    TT_TRY(check_ptr(packed, "packed"));
    TT_TRY(check_ptr(w_out, "w_out"));
    TT_TRY(check_align(packed, 16, "packed"));
    TT_TRY(check_align(w_out, 4, "w_out"));
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, "n"));
    TT_TRY(check_range(k, 1, TT_MAX_K_FP8, "k"));
    const F8Geom g = f8_geom(k);
    F8DequantArgs da{static_cast<const uint8_t *>(packed), g.stride, (int32_t)n, (int32_t)k,
                     (int32_t)g.scale_off, w_out, scale_out};
    tt_status st = launch("fp8 dequantize", k_f8_dequant,
                          dim3((unsigned)ceil_div(n, kF8TileRows), (unsigned)g.units), dim3(64), 0,
                          static_cast<hipStream_t>(stream), da);
    if (st == TT_OK) clear_error();
    return st;
}
