// device.h -- gfx950 device helpers shared by the kernels: E8M0 scales,
// the FP4 block dot products, activations and output conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"
#include "tt_internal.h"

namespace tt {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

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

// The 8 FP4 codes of one dword (code 2j in bits 8j..8j+3, code 2j+1 in bits
// 8j+4..8j+7) against 8 bf16 activations held as 4 packed pairs.  Each
// conversion turns one byte (two codes) into two exact bf16 values; the dot2
// multiplies them with the matching activation pair and accumulates in fp32.
__device__ __forceinline__ float fp4x8_dot_bf16(uint32_t c, uint4 x, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(
        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 0), as_bf16x2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(
        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 1), as_bf16x2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(
        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 2), as_bf16x2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(
        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 3), as_bf16x2(x.w), acc, false);
    return acc;
}

// One 32-element MX block (16 code bytes) against 32 bf16 activations
// (4 x 16 bytes), unscaled.  Two accumulators shorten the dependency chain.
__device__ __forceinline__ float fp4x32_dot_bf16(uint4 c, const uint4 *x) {
    float p0 = fp4x8_dot_bf16(c.x, x[0], 0.0f);
    float p1 = fp4x8_dot_bf16(c.y, x[1], 0.0f);
    p0 = fp4x8_dot_bf16(c.z, x[2], p0);
    p1 = fp4x8_dot_bf16(c.w, x[3], p1);
    return p0 + p1;
}

// The same block against fp32 activations (8 x 16 bytes).
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

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

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

// Stage n bf16 activations into LDS, zero-filling up to n_pad (both
// multiples of 8); 16-byte chunks, all threads of the block cooperate.
__device__ __forceinline__ void stage_bf16(uint16_t *dst, const uint16_t *src, int n,
                                           int n_pad, int tid, int nthreads) {
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
    uint4 *d = reinterpret_cast<uint4 *>(dst);
    for (int i = tid; i < n_pad / 8; i += nthreads)
        d[i] = (i < n / 8) ? s[i] : make_uint4(0, 0, 0, 0);
}

// Launch a kernel whose only parameter is an argument struct and report the
// launch's own status (not a stale error left by earlier runtime calls).
template <typename A>
tt_status launch(const char *what, void (*kernel)(A), dim3 grid, dim3 block, size_t lds,
                 hipStream_t stream, const A &args) {
    void *argv[] = {const_cast<A *>(&args)};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds,
                                   stream);
    if (e != hipSuccess) return fail(TT_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return TT_OK;
}

}  // namespace tt
