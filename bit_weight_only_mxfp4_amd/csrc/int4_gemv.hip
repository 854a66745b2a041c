// int4_gemv.hip -- grouped affine INT4 matvec for the attention projections
// (stardance page, "numerical drift & speedups": dense INT4 Q/K/V/O;
// "Implemented a huge list of fixes": affine INT4 with a partial last group):
//   y[b][r] = sum_g s[r][g] * sum_{k in g} (q[r][k] - z[r][g]) * x[b][k]
//
// Layout and grid follow the MXFP4 kernel: one workgroup per 16-row tile, KS
// waves splitting the groups, one 16-byte load per lane per unit (32 codes of
// one row; a unit is one 128-element group).  Decode: a code q becomes the
// bf16 number 128 + q by OR-ing it under the exponent pattern 0x4300 (exact),
// two at a time, and a dot2 accumulates (128 + q) * x in fp32.  Per 32-element
// piece the activations' plain sum X is staged once, so the group term is
//   s * (sum (128 + q) x - (128 + z) * X)  =  s * sum (q - z) x.
// The activations are staged in LDS with each 8-element group reordered as
// pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7), matching the nibble pairs one
// shift-and-mask extracts from a code dword.
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
};

constexpr int kI4PF = 8;

// (128 + q) x summed over the 8 codes of one dword; xg holds the reordered
// activation pairs of that 8-element group.
__device__ __forceinline__ float i4x8_dot(uint32_t c, uint4 xg, float acc) {
    const uint32_t m = 0x000F000Fu, bias = 0x43004300u;
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2((c & m) | bias), as_bf16x2(xg.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(((c >> 4) & m) | bias), as_bf16x2(xg.y), acc,
                                          false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(((c >> 8) & m) | bias), as_bf16x2(xg.z), acc,
                                          false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(((c >> 12) & m) | bias), as_bf16x2(xg.w), acc,
                                          false);
    return acc;
}

template <int KS, int NT>
__global__ __launch_bounds__(64 * KS) void k_int4_gemv(I4Args a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int kp = a.units * 128;  // padded K
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);                       // [NT][kp]
    float *xsum = reinterpret_cast<float *>(smem + (size_t)NT * kp * 2);     // [NT][kp/32]
    float *red = xsum + NT * (kp / 32);                                      // [KS][NT][16]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x, t0 = blockIdx.y * NT;
    const int nt = min(NT, a.batch - t0);

    // stage: one thread per (token, 32-element piece)
    const int pieces = kp / 32;
    for (int i = tid; i < NT * pieces; i += 64 * KS) {
        const int t = i / pieces, p = i % pieces;
        uint4 *dst = reinterpret_cast<uint4 *>(xs + t * kp + p * 32);
        float sum = 0.0f;
        const uint16_t *src = a.x + (int64_t)(t0 + t) * a.k;
#pragma unroll
        for (int g8 = 0; g8 < 4; ++g8) {
            uint32_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = p * 32 + g8 * 8 + j;
                v[j] = (t < nt && kk < a.k) ? src[kk] : 0u;
                sum += bf16_bits_to_f32(v[j]);
            }
            dst[g8] = make_uint4(v[0] | (v[4] << 16), v[1] | (v[5] << 16), v[2] | (v[6] << 16),
                                 v[3] | (v[7] << 16));
        }
        xsum[t * pieces + p] = sum;
    }
    __syncthreads();

    const int r = lane & 15, q = lane >> 4;
    const uint8_t *tb = a.w + (int64_t)tile * a.tile_stride;
    const int upw = (a.units + KS - 1) / KS;
    const int u0 = wave * upw, u1 = min(a.units, u0 + upw);
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    for (int kb = u0; kb < u1; kb += kI4PF) {
        uint4 c[kI4PF];
        uint32_t sz[kI4PF];
#pragma unroll
        for (int i = 0; i < kI4PF; ++i) {
            const int kk = kb + i;
            if (kk < u1) {
                const int off = kk * kUnitBytes +
                                ((kk == a.units - 1 && q >= a.qv_last) ? r * 16 : lane * 16);
                c[i] = *reinterpret_cast<const uint4 *>(tb + off);
                sz[i] = *reinterpret_cast<const uint32_t *>(tb + a.sz_off + (kk >> 2) * kGroupBytes +
                                                            r * 16 + (kk & 3) * 4);
            }
        }
#pragma unroll
        for (int i = 0; i < kI4PF; ++i) {
            const int kk = kb + i;
            if (kk < u1) {
                const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz[i] & 0xFFFFu));
                const float zb = 128.0f + (float)__builtin_bit_cast(_Float16, (uint16_t)(sz[i] >> 16));
                const int p = 4 * kk + q;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (t < nt) {
                        const uint4 *xg = reinterpret_cast<const uint4 *>(xs + t * kp + p * 32);
                        float d0 = i4x8_dot(c[i].x, xg[0], 0.0f);
                        float d1 = i4x8_dot(c[i].y, xg[1], 0.0f);
                        d0 = i4x8_dot(c[i].z, xg[2], d0);
                        d1 = i4x8_dot(c[i].w, xg[3], d1);
                        acc[t] = fmaf(s, fmaf(-zb, xsum[t * pieces + p], d0 + d1), acc[t]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        acc[t] += __shfl_xor(acc[t], 16);
        acc[t] += __shfl_xor(acc[t], 32);
    }
    if (KS > 1) {
        if (lane < 16)
#pragma unroll
            for (int t = 0; t < NT; ++t) red[(wave * NT + t) * 16 + lane] = acc[t];
        __syncthreads();
        if (wave != 0) return;
        if (lane < 16)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float v = red[t * 16 + lane];
#pragma unroll
                for (int w = 1; w < KS; ++w) v += red[(w * NT + t) * 16 + lane];
                acc[t] = v;
            }
    }
    const int row = tile * 16 + lane;
    if (lane < 16 && row < a.n)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < nt) store_out(a.y, (int64_t)(t0 + t) * a.n + row, acc[t], a.y_bf16);
}

namespace {

int pick_ks(int units) {
    if (units >= 48) return 8;
    if (units >= 24) return 4;
    if (units >= 12) return 2;
    return 1;
}

constexpr size_t kLdsBudget = 64 * 1024;

size_t lds_bytes(int units, int nt, int ks) {
    const size_t kp = (size_t)units * 128;
    return (size_t)nt * kp * 2 + (size_t)nt * (kp / 32) * 4 + (size_t)ks * nt * 64;
}

template <int NT>
tt_status launch_nt(const I4Args &a, int ks, hipStream_t s) {
    const size_t lds = lds_bytes(a.units, NT, ks);
    dim3 grid(a.ntiles, (a.batch + NT - 1) / NT);
    const char *what = "int4 gemv";
    switch (ks) {
        case 1: return launch(what, k_int4_gemv<1, NT>, grid, dim3(64), lds, s, a);
        case 2: return launch(what, k_int4_gemv<2, NT>, grid, dim3(128), lds, s, a);
        case 4: return launch(what, k_int4_gemv<4, NT>, grid, dim3(256), lds, s, a);
        default: return launch(what, k_int4_gemv<8, NT>, grid, dim3(512), lds, s, a);
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
    const int ks = pick_ks(a.units);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // tokens per weight pass: as many as the batch needs, as LDS allows
    int nt = batch == 1 ? 1 : batch == 2 ? 2 : batch <= 4 ? 4 : 8;
    while (nt > 1 && lds_bytes(a.units, nt, ks) > kLdsBudget) nt /= 2;
    tt_status st;
    if (nt == 1)
        st = launch_nt<1>(a, ks, s);
    else if (nt == 2)
        st = launch_nt<2>(a, ks, s);
    else if (nt == 4)
        st = launch_nt<4>(a, ks, s);
    else
        st = launch_nt<8>(a, ks, s);
    if (st == TT_OK) clear_error();
    return st;
}
