// device.h -- gfx950 device helpers shared by the kernels: E8M0 scales,
// the FP4 block dot products, activations and output conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "layout.h"
#include "tt_internal.h"

namespace tt {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Cache-policy operand of the buffer loads that stream bytes read once per
// call (packed weights, their scales and postscales, the KV cache): the
// instruction's non-temporal bit (`nt`).  Activations, which every workgroup
// re-reads, keep the default policy.  On MI355X a plain read of 17.7 or
// 24 MB ran 7-10 % faster with it; the scope bits (sc0, sc1) made no
// difference.  The INT4 kernel keeps the default policy: with the hint its
// Phi-4 O projection ran 6 % slower and its QKV projection no faster.
constexpr int kStreamPolicy = 2;

// A kernel argument held in scalar registers from this point on.  Arguments
// past the preloaded ones are otherwise read from argument memory where they
// are used; after a workgroup barrier that read adds a memory round trip to
// the end of the kernel.  Place it after the kernel's streaming loads are
// issued, so the read overlaps them.
template <typename T>
__device__ __forceinline__ T hold_sgpr(T v) {
    asm volatile("" : "+s"(v));
    return v;
}

// E8M0 scale byte -> fp32 2^(e-127).  Byte 0 is the fp32 subnormal 2^-127,
// byte 255 is NaN; every other byte is a normal power of two.
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
    uint32_t b = e << 23;
    b = (e == 0u) ? 0x00400000u : b;
    b = (e == 255u) ? 0x7FC00000u : b;
    return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) {
    return __builtin_bit_cast(bf16x2_t, v);
}

// One 32-element MX block (16 code bytes: code 2j in bits 8j..8j+3, code
// 2j+1 in bits 8j+4..8j+7 of its byte) against fp32 activations (8 x 16
// bytes), unscaled: the hardware FP4 conversion gives exact fp32 pairs, one
// FMA per element, two accumulators to shorten the dependency chain.
__device__ __forceinline__ float fp4x8_dot_f32(uint32_t c, float4 xa, float4 xb, float acc) {
    f32x2_t v;
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    acc = fmaf(v.x, xa.x, acc);
    acc = fmaf(v.y, xa.y, acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    acc = fmaf(v.x, xa.z, acc);
    acc = fmaf(v.y, xa.w, acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    acc = fmaf(v.x, xb.x, acc);
    acc = fmaf(v.y, xb.y, acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    acc = fmaf(v.x, xb.z, acc);
    acc = fmaf(v.y, xb.w, acc);
    return acc;
}

__device__ __forceinline__ float fp4x32_dot_f32(uint4 c, const float4 *x) {
    float p0 = fp4x8_dot_f32(c.x, x[0], x[1], 0.0f);
    float p1 = fp4x8_dot_f32(c.y, x[2], x[3], 0.0f);
    p0 = fp4x8_dot_f32(c.z, x[4], x[5], p0);
    p1 = fp4x8_dot_f32(c.w, x[6], x[7], p1);
    return p0 + p1;
}

// Eight FP4 codes of one dword scaled by `sc` into an 8 x bf16 MFMA operand
// (exact while the scaled values are normal bf16 numbers).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t c, float sc) {
    u32x4_t v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0));
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1));
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2));
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3));
    return __builtin_bit_cast(bf16x8_t, v);
}

// Cross-lane sums over lane pairs (l, l ^ 8), (l, l ^ 16), (l, l ^ 32) without
// LDS permutes: a DPP rotate by 8 within each row of 16 lanes, and the gfx950
// row-swap instructions (v_permlane16_swap / v_permlane32_swap exchange odd
// rows with even rows, resp. the upper half-wave with the lower).  Both lanes
// of a pair get the same bits.  All 64 lanes must be active.
__device__ __forceinline__ float sum_xor8(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF,
                                             false));
}
// (The pair of results is bit-cast as a whole vector: a bit_cast of one
// element of an ext-vector value is miscompiled to element 0.)
__device__ __forceinline__ float sum_xor16(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const f32x2_t r =
        __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane16_swap(b, b, false, false));
    return r.x + r.y;
}
__device__ __forceinline__ float sum_xor32(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const f32x2_t r =
        __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane32_swap(b, b, false, false));
    return r.x + r.y;
}

// silu(z) = z / (1 + e^-z) from the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32): within a few units in the last place of the
// fp32 quotient, against some 25 instructions for expf and a rounded divide
// in the epilogue every output waits for.  Limits: z = +inf gives +inf,
// z -> -inf gives -0 (e^-z overflows to inf, its reciprocal is 0), NaN
// stays NaN.
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ void store_out(void *out, int64_t i, float v, int bf16) {
    if (bf16)
        static_cast<uint16_t *>(out)[i] = f32_to_bf16_bits(v);
    else
        static_cast<float *>(out)[i] = v;
}

// ---- scaled FP4 x FP8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) -----------
// A (16 x 128, FP4 E2M1, 4 registers): lane l holds row l % 16, elements
// 32 (l / 16) .. +31 -- exactly one packed tile unit as loaded; A scale: the
// lane's E8M0 byte for that 32-element piece.  B (128 x 16, FP8 E4M3, 8
// registers): lane (column c = l % 16, group g = l / 16) holds elements
// 16g .. 16g+15 in its first four registers and 64+16g .. +15 in the next
// four; B scale of lane (c, g): the E8M0 byte of elements 32g .. 32g+31.
// Output: lane (c, g) holds rows 4g .. 4g+3 of column c.  (Layouts measured
// on the device.)  Activations enter as two E4M3 parts per 32-element block,
//   x = 2^(E-7) hi + 2^(E-11) lo,   E = the block's largest bf16 exponent,
// exact for every element of magnitude >= 2^(E-13) (hi carries the top 4
// of the 8 significant bits, lo the rest) and to within 2^(E-21) below.
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

// Largest bf16 exponent field among the 8 elements of a 16-byte chunk.
__device__ __forceinline__ uint32_t bf16x8_max_exp(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max((w[i] >> 7) & 255u, (w[i] >> 23) & 255u));
    return m;
}

// hi and lo E4M3 parts of 4 bf16 values (2 dwords) times mult = 2^(127 - sh).
__device__ __forceinline__ void split4(uint32_t w0, uint32_t w1, float mult, uint32_t *hi,
                                       uint32_t *lo) {
    const float v0 = bf16_bits_to_f32(w0 & 0xFFFFu) * mult, v1 = bf16_bits_to_f32(w0 >> 16) * mult;
    const float v2 = bf16_bits_to_f32(w1 & 0xFFFFu) * mult, v3 = bf16_bits_to_f32(w1 >> 16) * mult;
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, h, true);
    const f32x2_t b01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
    const f32x2_t b23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
    int l = __builtin_amdgcn_cvt_pk_fp8_f32((v0 - b01.x) * 16.0f, (v1 - b01.y) * 16.0f, 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32((v2 - b23.x) * 16.0f, (v3 - b23.y) * 16.0f, l, true);
    *hi = (uint32_t)h;
    *lo = (uint32_t)l;
}

// The two E4M3 parts of one 16-byte chunk (8 bf16) of a 32-element block
// whose four chunks sit in four consecutive lanes (their largest exponent is
// shared through two DPP quad swaps, so all 64 lanes must take part).
// Returns the hi part's E8M0 byte, 2^(E-7) kept in [5, 254]; the lo part's
// byte is 4 less.  Zero chunks give zero parts.
__device__ __forceinline__ uint32_t split_chunk(uint4 v, uint2 *hi, uint2 *lo) {
    uint32_t e = bf16x8_max_exp(v);
    e = max(e, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0xB1, 0xF, 0xF, false));
    e = max(e, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x4E, 0xF, 0xF, false));
    const uint32_t sh = min(max(e, 12u) - 7u, 254u);
    const float mult = __builtin_bit_cast(float, (254u - sh) << 23);  // 2^(127 - sh)
    split4(v.x, v.y, mult, &hi->x, &lo->x);
    split4(v.z, v.w, mult, &hi->y, &lo->y);
    return sh;
}

// One scaled MFMA, FP4 A by FP8 B; byte sel of both scale dwords (the
// selector must be a constant: the unrolled unit index folds the switch).
template <int SEL>
__device__ __forceinline__ f32x4_t mfma_fp4_fp8_sel(i32x8_t A, i32x8_t B, f32x4_t C, uint32_t sa,
                                                    uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, 4, 0, SEL, (int)sa, SEL,
                                                            (int)sb);
}
__device__ __forceinline__ f32x4_t mfma_fp4_fp8(int sel, i32x8_t A, i32x8_t B, f32x4_t C,
                                                uint32_t sa, uint32_t sb) {
    switch (sel) {
        case 0: return mfma_fp4_fp8_sel<0>(A, B, C, sa, sb);
        case 1: return mfma_fp4_fp8_sel<1>(A, B, C, sa, sb);
        case 2: return mfma_fp4_fp8_sel<2>(A, B, C, sa, sb);
        default: return mfma_fp4_fp8_sel<3>(A, B, C, sa, sb);
    }
}

// Launch a kernel and report the launch's own status (not a stale error
// left by earlier runtime calls).  The streaming kernels take what they need
// before their first weight load as leading scalar parameters: the library is
// built to preload the first 16 dwords of kernel arguments into scalar
// registers at wave launch, so those values cost no memory round trip.  The
// rest comes in one argument struct, read after the weight loads are issued.
template <typename T> struct same_type { using type = T; };
template <typename... P>
tt_status launch(const char *what, void (*kernel)(P...), dim3 grid, dim3 block, size_t lds,
                 hipStream_t stream, const typename same_type<P>::type &...args) {
    void *argv[] = {const_cast<void *>(static_cast<const void *>(&args))...};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds,
                                   stream);
    if (e != hipSuccess) return fail(TT_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return TT_OK;
}

// Raise a kernel's dynamic LDS limit to the 160 KiB of a gfx950 CU, once
// per device.  Several host threads may call this at once: the per-device
// flags are one atomic word, and the attribute call is idempotent, so two
// threads that both find the flag clear both make it, with the same effect.
// Kernel is the kernel function itself (one flag word per kernel).
constexpr int kLdsLimitBytes = 160 * 1024;
template <auto Kernel>
tt_status raise_lds_limit(const char *what) {
    static std::atomic<uint64_t> raised{0};  // bit d: done on device d
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(TT_E_HIP, "%s: no usable current device", what);
    const uint64_t bit = uint64_t{1} << dev;
    if (raised.load(std::memory_order_acquire) & bit) return TT_OK;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(Kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLdsLimitBytes) != hipSuccess)
        return fail(TT_E_HIP, "%s: cannot raise the LDS limit", what);
    raised.fetch_or(bit, std::memory_order_release);
    return TT_OK;
}

}  // namespace tt
