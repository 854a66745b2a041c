// int4_gemv.hip -- grouped affine INT4 matvec for the attention projections
// (stardance page, "numerical drift & speedups": dense INT4 Q/K/V/O;
// "Implemented a huge list of fixes": affine INT4 with a partial last group):
//   y[b][r] = sum_g s[r][g] * sum_{k in g} (q[r][k] - z[r][g]) * x[b][k]
//
// Layout and grid follow the MXFP4 kernel: one workgroup per 16-row tile, ks
// waves splitting the groups, one 16-byte load per lane per unit (32 codes of
// one row; a unit is one 128-element group), all of a wave's loads in flight
// before the activations are staged.  Decode: a code q becomes the
// bf16 number 128 + q by OR-ing it under the exponent pattern 0x4300 (exact),
// two at a time, and the bf16 matrix cores sum (128 + q) * x over each
// 128-element group in fp32 (the tile's 16 rows are the product's columns,
// the tokens its rows).  Per group the activations' plain sum X is staged
// once, so the group term is
//   s * (sum (128 + q) x - (128 + z) * X)  =  s * sum (q - z) x.
// The two sums are taken in different orders, so a group whose codes all
// equal its zero point would leave a rounding residue instead of 0; the
// packer stores a zero scale for such a group (its weights are all zero), so
// its term is exactly 0.
// The activations are staged in LDS with each 8-element group reordered as
// pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7), matching the nibble pairs one
// shift-and-mask extracts from a code dword; both operands of a product
// carry the same order, so each k slot meets its own activation.
#include "device.h"
#include "tt_internal.h"

namespace tt {

struct I4Args {
    const uint8_t *w;
    int64_t tile_stride;
    int32_t n, k, units, qv_last, sz_off, ntiles;
    const uint16_t *x;  // [batch][k]
    int32_t batch;
    void *y;            // [batch][n]
    int32_t y_bf16;
    int32_t ks;         // waves per tile
    int32_t xvec;       // x rows are 16-byte aligned (k % 8 == 0 and x aligned)
                        // and batch * k * 2 fits a buffer range
};

// Tuning: units (128-element groups) per wave; a tile uses at most 16 waves.
#ifndef TT_INT4_UPW
#define TT_INT4_UPW 4
#endif
constexpr int kOob = 0x7FFFFF00;  // buffer offset past every tile: loads return 0

// (x & m) | b, written in C so that the compiler sees every register it
// writes: it must space VALU writes from the matrix instructions still in
// flight on the same registers, and it cannot do that for inline assembly.
// With b held in a VGPR (see k_int4_gemv) this is one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t b) {
    return (x & m) | b;
}

__device__ __forceinline__ uint4 i4_load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void i4_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One workgroup per 16-row tile and NT tokens; wave p owns units
// [p * UPW, p * UPW + UPW).  Issue order per wave: the activations of its
// pieces, then each s|z group followed by its four code units.  Units past K
// read at an out-of-range buffer offset (zeros) and meet zero-padded
// activations and zero group sums, so they add exactly nothing.
// The argument struct with the leading kernel parameters written in (they
// are preloaded into scalar registers): everything read before the weight
// loads (the tile geometry follows from k), and the output, which the tail
// after the last barrier needs (read from argument memory there, it would
// add a memory round trip to the end of every call).
__device__ __forceinline__ I4Args i4_hot_args(I4Args a, const uint8_t *w, const uint16_t *x,
                                              int32_t k, int32_t batch, int32_t ks, int32_t n,
                                              void *y, int32_t y_bf16) {
    const I4Geom g = i4_geom(k);
    a.w = w;
    a.x = x;
    a.k = k;
    a.units = (int32_t)g.units;
    a.qv_last = (int32_t)g.qv_last;
    a.sz_off = (int32_t)g.sz_off;
    a.tile_stride = g.stride;
    a.batch = batch;
    a.ks = ks;
    a.n = n;
    a.y = y;
    a.y_bf16 = y_bf16;
    return a;
}

template <int UPW, int NT, bool XVEC>
__global__ __launch_bounds__(1024) void k_int4_gemv(const uint8_t *w, const uint16_t *x,
                                                    int32_t k, int32_t batch, int32_t ks_,
                                                    int32_t rows, void *y, int32_t y_bf16,
                                                    I4Args cold) {
    static_assert(UPW % 4 == 0 && UPW <= 16, "units per wave");
    const I4Args a = i4_hot_args(cold, w, x, k, batch, ks_, rows, y, y_bf16);
    extern __shared__ __align__(16) uint8_t smem[];
    const int ks = a.ks;
    const int kp = ks * UPW * 128;   // staged K per token, zero past a.k
    const int upk = kp / 128;        // staged units per token
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);                   // [NT][kp]
    float *xsum = reinterpret_cast<float *>(smem + (size_t)NT * kp * 2); // [NT][upk]
    float *red = xsum + NT * upk;                                        // [ks][NT][16]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = blockIdx.x, t0 = blockIdx.y * NT;
    const int nt = min(NT, a.batch - t0);

    // 1. activations: each wave fetches the slice of every token that its
    //    own units read (UPW * 128 elements, one 8-element group per lane
    //    per load), so no other wave waits on it.  Rows of 16-byte aligned x
    //    go out as straight-line buffer loads (zeros past the batch and past
    //    k); other rows take element loads.
    constexpr int XL = UPW / 4;  // loads per lane per token
    const int kw = wave * UPW * 128;  // first element of the wave's slice
    uint32_t xw[NT][XL][4];
    {
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.x), 0, XVEC ? a.batch * a.k * 2 : 0, 0x00020000);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bool tok_ok = t < nt;
#pragma unroll
            for (int j = 0; j < XL; ++j) {
                const int k0 = kw + (j * 64 + lane) * 8;
                if (XVEC) {
                    const bool ok = tok_ok && k0 < a.k;
                    const uint4 v = i4_load16(xr, ok ? ((t0 + t) * a.k + k0) * 2 : kOob);
                    xw[t][j][0] = v.x;
                    xw[t][j][1] = v.y;
                    xw[t][j][2] = v.z;
                    xw[t][j][3] = v.w;
                } else {
                    const uint16_t *src = a.x + (int64_t)(t0 + t) * a.k + k0;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t lo = (tok_ok && k0 + 2 * d < a.k) ? src[2 * d] : 0u;
                        const uint32_t hi = (tok_ok && k0 + 2 * d + 1 < a.k) ? src[2 * d + 1] : 0u;
                        xw[t][j][d] = lo | (hi << 16);
                    }
                }
            }
        }
    }

    // keep the activation loads ahead of the weights (completion is in
    // order: the staging below then waits for the activations only)
    __builtin_amdgcn_sched_barrier(0);

    // 2. weights
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.w + (int64_t)tile * a.tile_stride), 0, (int)a.tile_stride,
        0x00020000);
    const int r = lane & 15, q = lane >> 4;
    const int u0 = wave * UPW;
    const int n = max(0, min(UPW, a.units - u0));
    uint4 c[UPW];
    uint4 szv[UPW / 4];
    const int voff = u0 * kUnitBytes + lane * 16;
    const int soff = a.sz_off + (u0 >> 2) * kGroupBytes + r * 16;
#pragma unroll
    for (int g = 0; g < UPW / 4; ++g) {
        szv[g] = i4_load16(rs, 4 * g < n ? soff + g * kGroupBytes : kOob);
#pragma unroll
        for (int i = 4 * g; i < 4 * g + 4; ++i)
            c[i] = i4_load16(rs, i < n ? voff + i * kUnitBytes : kOob);
    }

    // 3. the wave's slice to LDS: 8-element groups reordered as (x0,x4)
    //    (x1,x5) (x2,x6) (x3,x7), and the plain sum of each 128-element group
    //    (the 16 lanes of a group add theirs with two DPP quad swaps and two
    //    row rotates, in a fixed order).  Only
    //    this wave reads the slice back, and a wave's LDS accesses complete in
    //    order, so no barrier is needed.
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const uint32_t w0 = xw[t][j][0], w1 = xw[t][j][1];
            const uint32_t w2 = xw[t][j][2], w3 = xw[t][j][3];
            // elements e0..e7 = lo(w0) hi(w0) lo(w1) hi(w1) lo(w2) hi(w2) lo(w3) hi(w3)
            *reinterpret_cast<uint4 *>(xs + t * kp + kw + (j * 64 + lane) * 8) =
                make_uint4((w0 & 0xFFFFu) | (w2 << 16), (w0 >> 16) | (w2 & 0xFFFF0000u),
                           (w1 & 0xFFFFu) | (w3 << 16), (w1 >> 16) | (w3 & 0xFFFF0000u));
            float sum = (bf16_bits_to_f32(w0 & 0xFFFFu) + bf16_bits_to_f32(w0 >> 16)) +
                        (bf16_bits_to_f32(w1 & 0xFFFFu) + bf16_bits_to_f32(w1 >> 16)) +
                        (bf16_bits_to_f32(w2 & 0xFFFFu) + bf16_bits_to_f32(w2 >> 16)) +
                        (bf16_bits_to_f32(w3 & 0xFFFFu) + bf16_bits_to_f32(w3 >> 16));
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 0, __builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF,
                                                 false));
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 0, __builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF,
                                                 false));
            // the four pieces of a unit (16 lanes): rotate by 4, then by 8
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 0, __builtin_bit_cast(int, sum), 0x124, 0xF, 0xF,
                                                 false));
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 0, __builtin_bit_cast(int, sum), 0x128, 0xF, 0xF,
                                                 false));
            if ((lane & 15) == 0) xsum[t * upk + kw / 128 + j * 4 + (lane >> 4)] = sum;
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

    // 4. each unit on the matrix cores (v_mfma_f32_16x16x32_bf16, one
    //    product per code dword): B = the lane's own codes decoded to
    //    128 + q (column = tile row r, k block = piece q), A = token
    //    l % 16's activations of the same piece in the same reordered
    //    element order (rows past NT read token NT - 1; their outputs are
    //    never used).  C lane (row r, group g) then holds the unit's
    //    sum of (128 + q) x for tokens 4g .. 4g+3, and the group's affine
    //    correction is applied to it: s (C - (128 + z) sum x).
    const int ta = min(r, NT - 1);
    f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // the bias 0x4300 (bf16 128.0) in both halves, in a VGPR whose value the
    // compiler does not fold into each use (a VOP3 op reads one scalar, and
    // the nibble mask takes it); set once, before any matrix instruction
    uint32_t bias;
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias));
    const uint32_t nib = 0x000F000Fu;
    // the group sums of the wave's units for this lane's tokens, read before
    // the first unit (16 bytes per four units) so that no unit waits on an
    // LDS round trip of its own (measured: QKV 5.59 -> 5.44 us)
    float xsv[4][UPW];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e >= NT) break;
        const int t = min(4 * q + e, NT - 1);
#pragma unroll
        for (int i4 = 0; i4 < UPW / 4; ++i4) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t *>(xsum + t * upk + u0 + 4 * i4);
#pragma unroll
            for (int j = 0; j < 4; ++j) xsv[e][4 * i4 + j] = v[j];
        }
    }
    // the activation operands of unit i + 1 are read from LDS while unit i
    // runs on the matrix cores
    const uint4 *xgb = reinterpret_cast<const uint4 *>(xs + ta * kp + (4 * u0 + q) * 32);
    uint4 xcur[4], xnext[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) xcur[m] = xgb[m];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const uint32_t sz = (i & 3) == 0 ? szv[i >> 2].x
                          : (i & 3) == 1 ? szv[i >> 2].y
                          : (i & 3) == 2 ? szv[i >> 2].z : szv[i >> 2].w;
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xFFFFu));
        const float zb = 128.0f + (float)__builtin_bit_cast(_Float16, (uint16_t)(sz >> 16));
        if (i + 1 < UPW) {
#pragma unroll
            for (int m = 0; m < 4; ++m) xnext[m] = xgb[(i + 1) * 16 + m];
        }
        const uint32_t cw[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
        f32x4_t cu = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint4 wb = make_uint4(and_or(cw[m], nib, bias), and_or(cw[m] >> 4, nib, bias),
                                        and_or(cw[m] >> 8, nib, bias),
                                        and_or(cw[m] >> 12, nib, bias));
            cu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xcur[m]),
                                                         __builtin_bit_cast(bf16x8_t, wb), cu, 0,
                                                         0, 0);
        }
        if (i + 1 < UPW) {
#pragma unroll
            for (int m = 0; m < 4; ++m) xcur[m] = xnext[m];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * q + e;
            if (t < NT)
                acc[e] = fmaf(s, fmaf(-zb, xsv[e][i], cu[e]), acc[e]);
        }
    }
    if (ks > 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * q + e < NT) red[(wave * NT + 4 * q + e) * 16 + r] = acc[e];
        i4_lds_barrier();
        if (wave != 0) return;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * q + e;
            if (t < NT) {
                float v = red[t * 16 + r];
                for (int w = 1; w < ks; ++w) v += red[(w * NT + t) * 16 + r];
                acc[e] = v;
            }
        }
    }
    const int row = tile * 16 + r;
    if (row < a.n)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * q + e;
            if (t < NT && t < nt) store_out(a.y, (int64_t)(t0 + t) * a.n + row, acc[e], a.y_bf16);
        }
}

namespace {

constexpr size_t kLdsBudget = 64 * 1024;

size_t lds_bytes(int ks, int upw, int nt) {
    const size_t kp = (size_t)ks * upw * 128;
    return (size_t)nt * kp * 2 + (size_t)nt * (kp / 128) * 4 + (size_t)ks * nt * 64;
}

template <int UPW, int NT>
tt_status launch_i4(I4Args a, hipStream_t s) {
    a.ks = (int32_t)ceil_div(a.units, UPW);
    dim3 grid(a.ntiles, (a.batch + NT - 1) / NT);
    const size_t lds = lds_bytes(a.ks, UPW, NT);
    return a.xvec ? launch("int4 gemv", k_int4_gemv<UPW, NT, true>, grid, dim3(64 * a.ks), lds, s,
                           a.w, a.x, a.k, a.batch, a.ks, a.n, a.y, a.y_bf16, a)
                  : launch("int4 gemv", k_int4_gemv<UPW, NT, false>, grid, dim3(64 * a.ks), lds, s,
                           a.w, a.x, a.k, a.batch, a.ks, a.n, a.y, a.y_bf16, a);
}

template <int UPW>
tt_status launch_upw(const I4Args &a, hipStream_t s) {
    // tokens per weight pass: as many as the batch needs, as LDS allows
    const int ks = (int)ceil_div(a.units, UPW);
    int nt = a.batch == 1 ? 1 : a.batch == 2 ? 2 : a.batch <= 4 ? 4 : 8;
    while (nt > 1 && lds_bytes(ks, UPW, nt) > kLdsBudget) nt /= 2;
    switch (nt) {
        case 1: return launch_i4<UPW, 1>(a, s);
        case 2: return launch_i4<UPW, 2>(a, s);
        case 4: return launch_i4<UPW, 4>(a, s);
        default: return launch_i4<UPW, 8>(a, s);
    }
}

}  // namespace
}  // namespace tt

using namespace tt;

extern "C" tt_status tt_int4_gemv(const void *w_packed, int64_t n, int64_t k, int64_t group,
                                  const void *x, int64_t batch, void *y, int32_t y_dtype,
                                  void *stream) {
    TT_TRY(check_ptr(w_packed, "w_packed"));
    TT_TRY(check_ptr(x, "x"));
    TT_TRY(check_ptr(y, "y"));
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, "n"));
    TT_TRY(check_range(k, 2, TT_MAX_K, "k"));
    if (k % 2) return fail(TT_E_SHAPE, "k = %lld is odd", (long long)k);
    if (group != TT_INT4_GROUP)
        return fail(TT_E_SHAPE, "group = %lld; only %d is supported", (long long)group,
                    TT_INT4_GROUP);
    TT_TRY(check_range(batch, 1, TT_MAX_BATCH, "batch"));
    TT_TRY(check_dtype(y_dtype, "y_dtype"));
    TT_TRY(check_align(w_packed, 16, "w_packed"));
    TT_TRY(check_align(x, 2, "x"));
    TT_TRY(check_align(y, y_dtype == TT_F32 ? 4 : 2, "y"));
    const I4Geom g = i4_geom(k);
    I4Args a;
    a.w = static_cast<const uint8_t *>(w_packed);
    a.tile_stride = g.stride;
    a.n = (int32_t)n;
    a.k = (int32_t)k;
    a.units = (int32_t)g.units;
    a.qv_last = (int32_t)g.qv_last;
    a.sz_off = (int32_t)g.sz_off;
    a.ntiles = (int32_t)ceil_div(n, 16);
    a.x = static_cast<const uint16_t *>(x);
    a.batch = (int32_t)batch;
    a.y = y;
    a.y_bf16 = y_dtype == TT_BF16;
    a.xvec = (k % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
             batch * k * 2 < (int64_t)kOob;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int upw = TT_INT4_UPW;
    while (ceil_div(a.units, upw) > 16) upw += 4;
    tt_status st;
    switch (upw) {
        case 4: st = launch_upw<4>(a, s); break;
        case 8: st = launch_upw<8>(a, s); break;
        case 12: st = launch_upw<12>(a, s); break;
        case 16: st = launch_upw<16>(a, s); break;
        default: return fail(TT_E_SHAPE, "k = %lld needs more than 8 waves per tile", (long long)k);
    }
    if (st == TT_OK) clear_error();
    return st;
}
