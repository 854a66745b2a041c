/*
 * tt.h -- weight-only MXFP4 / INT4 single-token decode projections for AMD
 * Instinct MI355X (gfx950).  C ABI of libtt.so.
 *
 * What the calls compute follows the ThinTensor developer logs:
 *   - page kerbin.cskartikey.dev/@satvikhardat, "Dev Log #4 -- 91-96 tok/s
 *     with Selective MXFP4": MXFP4 on the MLP gate/up projections with a row
 *     postscale; out[r] = silu(ps_g[r] (Wg x)[r]) * (ps_u[r] (Wu x)[r]) over
 *     4-bit codes with one power-of-two scale per 32 weights and bf16 x, the
 *     postscale multiplying the finished row sum (section "Where Blackwell
 *     helps");
 *   - same page, "Dev Log #2 -- Converting SafeTensors Into .thin": a dense
 *     MLP needs a gated activation; an MoE model has router and expert stages;
 *   - page stardance.hackclub.com/projects/29750, "numerical drift &
 *     speedups": a matvec over the selected (routed) experts in MXFP4 and
 *     dense INT4 Q/K/V/O projections; "Implemented a huge list of fixes":
 *     affine INT4 with a partial last group; "ThinTensor Improvements":
 *     exact routing.
 * The MXFP4 bit layout is the OCP Microscaling Formats (MX) v1.0 one: FP4
 * E2M1 elements, one E8M0 scale per 32 consecutive elements along K.
 *
 * Canonical (caller-side) formats, all row-major, used by the packers:
 *   MXFP4 matrix W[N][K], K % 32 == 0:
 *     codes  u8[N][K/2]   element 2j in the low nibble of byte j, 2j+1 high
 *     scales u8[N][K/32]  E8M0: 2^(e-127); 0xFF is NaN
 *     ps     f32[N]       row postscale, multiplies the full-K sum (NULL = 1)
 *   INT4 matrix W[N][K], K even, group g = 128 consecutive k of one row:
 *     q u8[N][K/2] (same nibble order, values 0..15), s and z IEEE binary16
 *     bit patterns u16[N][ceil(K/128)], w = s * (q - z).
 *   Activations x: bf16 bit patterns [B][K]; outputs f32 or bf16 [B][N].
 *
 * Conventions for every call:
 *   - Return value: TT_OK or a negative tt_status; tt_last_error() then holds
 *     a message (thread-local).  On error nothing is launched or written.
 *   - Memory: every buffer is owned by the caller.  The library never
 *     allocates, frees, copies between host and device or synchronises.
 *     Device calls take device pointers; packers take host pointers.
 *   - Device calls enqueue kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and return.  Faults of the kernels themselves surface
 *     at the caller's next synchronisation.  Results are deterministic
 *     (fixed summation order, no floating-point atomics).  The calls are
 *     safe under stream capture.
 *   - Alignment: packed weights, x and h must be 16-byte aligned; other
 *     device buffers need the natural alignment of their element type.
 *   - Packed weights use a private tiled layout produced by the tt_pack_*
 *     functions; size it with the matching *_pack_bytes query.  An expert
 *     bank is n_experts packs laid end to end, each of the queried size.
 */
#ifndef TT_H
#define TT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TT_ABI_VERSION 1

typedef int32_t tt_status;
enum {
    TT_OK = 0,
    TT_E_NULL = -1,   /* a required pointer is NULL */
    TT_E_SHAPE = -2,  /* a size is out of range or not a multiple it must be */
    TT_E_ALIGN = -3,  /* a pointer is not aligned as required */
    TT_E_DTYPE = -4,  /* unknown element-type code */
    TT_E_SIZE = -5,   /* destination buffer smaller than the queried size */
    TT_E_RANGE = -6,  /* a value does not fit its format (INT4 scale) */
    TT_E_HIP = -7     /* the HIP runtime refused a launch */
};

/* Element types of activations and outputs. */
enum { TT_F32 = 0, TT_BF16 = 1 };

/* Weight formats for tt_format_info. */
enum { TT_FMT_MXFP4 = 0, TT_FMT_INT4_AFFINE = 1 };
/* Scale kinds reported by tt_format_info. */
enum { TT_SCALE_E8M0 = 0, TT_SCALE_F16 = 1 };

/* Limits enforced by the calls (TT_E_SHAPE beyond them). */
#define TT_MAX_K 16384        /* reduction dimension (hidden / inter) */
#define TT_MAX_ROWS (1 << 20) /* output rows */
#define TT_MAX_BATCH 32       /* tokens per call */
#define TT_MAX_EXPERTS 256
#define TT_MAX_TOPK 8
#define TT_INT4_GROUP 128
#define TT_MAX_K_FP8 32768    /* reduction dimension of the FP8 matvec */
#define TT_MAX_ATTN_T (1 << 20) /* cached positions of one attention call */

/* Library version of this header's ABI. */
int32_t tt_abi_version(void);
/* Message of the last failed call on this thread ("" if none). */
const char *tt_last_error(void);
/* Name of a status code. */
const char *tt_status_str(tt_status s);

/*
 * Honest format description ("Dev Log #4", section "Honest quantization
 * descriptors": bits, group size, scale type and zero point are stated, never
 * implied).  MXFP4: 4 bits, group 32, E8M0 scale, no zero point.  INT4:
 * 4 bits, group 128, binary16 scale, binary16 zero point.  Any output
 * pointer may be NULL.  TT_E_DTYPE for an unknown format.
 */
tt_status tt_format_info(int32_t format, int32_t *bits, int32_t *group,
                         int32_t *scale_kind, int32_t *has_zero);

/* ---------------------------------------------------------------------- */
/* Host-side packers (pure CPU, caller-owned buffers, no allocation)       */
/* ---------------------------------------------------------------------- */

/* Bytes of a packed MXFP4 matrix of n rows and k columns (k % 32 == 0),
 * or a negative tt_status for an invalid shape. */
int64_t tt_mxfp4_matrix_pack_bytes(int64_t n, int64_t k);

/* Pack one canonical MXFP4 matrix (codes, scales, ps as described above;
 * ps may be NULL for all ones) into dst, which holds dst_bytes >=
 * tt_mxfp4_matrix_pack_bytes(n, k).  Used for the expert down projections. */
tt_status tt_pack_mxfp4_matrix(const uint8_t *codes, const uint8_t *scales,
                               const float *ps, int64_t n, int64_t k,
                               void *dst, int64_t dst_bytes);

/* Bytes of a packed gate/up pair (inter rows each, hidden columns). */
int64_t tt_mxfp4_gateup_pack_bytes(int64_t inter, int64_t hidden);

/* Pack a gate matrix and an up matrix (each canonical MXFP4 [inter][hidden]
 * with its own postscale) so that one pass reads both rows of every output
 * feature. */
tt_status tt_pack_mxfp4_gateup(const uint8_t *g_codes, const uint8_t *g_scales,
                               const float *g_ps,
                               const uint8_t *u_codes, const uint8_t *u_scales,
                               const float *u_ps,
                               int64_t inter, int64_t hidden,
                               void *dst, int64_t dst_bytes);

/*
 * MXFP4 quantizer (the stardance page, "ThinTensor Improvements": MXFP4
 * quantizers; the conversion rule is the OCP MX v1.0 specification's, for a
 * vector of scalars to an MX block).  For every row and every block of 32
 * consecutive k (k a multiple of 32):
 *   e      = floor(log2(max |w|)) - 2, clamped to [-127, 127]; an all-zero
 *            block takes e = -127 (scale byte 0)
 *   scale  = E8M0 byte e + 127
 *   code_k = nearest FP4 E2M1 value of w_k / 2^e, ties to the even code,
 *            magnitudes above 6 clamped to 6, sign kept (-0 is code 8)
 * codes are written [n][k/2] (element 2j in the low nibble of byte j),
 * scales [n][k/32].  When ps is not NULL it receives the row postscale the
 * Dev Log #4 profile enables ("MXFP4 row postscale: enabled"); the pages do
 * not say how it is chosen, so it is the least-squares fit of the row,
 * ps = <w, d> / <d, d> over the decoded row d (fp64 sums in k order, rounded
 * to fp32; 1 when d is zero).  Host function; all buffers are host memory
 * owned by the caller.  TT_E_RANGE (nothing written) if an input is not
 * finite.
 */
tt_status tt_quantize_mxfp4(const float *w, int64_t n, int64_t k, uint8_t *codes,
                            uint8_t *scales, float *ps);

/*
 * Affine INT4 quantizer ("Implemented a huge list of fixes": affine INT4 with
 * a correct partial last group).  For every row and every group of `group`
 * (= 128) consecutive k -- the last group holding what is left of k -- over
 * that group's elements only, computed in fp64 from the fp32 inputs:
 *   lo = min(0, min w), hi = max(0, max w)
 *   s  = binary16 nearest-even of (hi - lo) / 15; s = 1 if that is 0
 *   z  = clamp(nearest-even(-lo / s), 0, 15)
 *   q  = clamp(nearest-even(w / s) + z, 0, 15)
 * q is written packed [n][k/2], s and z as binary16 bit patterns [n][G].
 * TT_E_RANGE if some s overflows binary16; k must be even.
 */
tt_status tt_quantize_int4_affine(const float *w, int64_t n, int64_t k,
                                  int64_t group, uint8_t *q, uint16_t *s,
                                  uint16_t *z);

/* Bytes of a packed INT4 matrix. */
int64_t tt_int4_pack_bytes(int64_t n, int64_t k, int64_t group);

/* Pack a canonical INT4 matrix (q, s, z) into dst.  A group whose codes all
 * equal its zero point (all of its weights are zero) is stored with a zero
 * scale of the same sign: the decoded weights are the same bits, and the
 * matvec then adds exactly 0 for that group. */
tt_status tt_pack_int4(const uint8_t *q, const uint16_t *s, const uint16_t *z,
                       int64_t n, int64_t k, int64_t group,
                       void *dst, int64_t dst_bytes);

/* ---------------------------------------------------------------------- */
/* Device calls                                                            */
/* ---------------------------------------------------------------------- */

/*
 * MXFP4 gate/up fused with SwiGLU ("Dev Log #4", "Where Blackwell helps";
 * "Dev Log #2" gated activation):
 *   g[b][r] = ps_g[r] * sum_k Wg[r][k] x[b][k]
 *   u[b][r] = ps_u[r] * sum_k Wu[r][k] x[b][k]
 *   out[b][r] = silu(g) * u,   silu(z) = z / (1 + e^-z)
 * w_gu: packed by tt_pack_mxfp4_gateup; x: bf16 [batch][hidden];
 * out: [batch][inter] of out_dtype (TT_F32 or TT_BF16, nearest-even).
 * 1 <= batch <= 32; hidden % 32 == 0, hidden <= TT_MAX_K.
 * Numerics.  Batch 1 and 2 run on the gfx950 scaled FP4 x FP8 matrix
 * instruction: weights and E8M0 scales as stored, each bf16 activation
 * carried exactly as two E4M3 parts (elements far below their block's
 * largest lose bits below 2^(E-21)), every product exact; the instruction
 * adds each 128-element block's products with a limited alignment width
 * before its fp32 accumulator, so a block whose products span many binades
 * is summed less exactly than in fp32.  Measured with products spread over
 * up to 2^43 inside every block at K = 16384: at most 0.4 % of the
 * 2e-3 * sum |w x| bound (random configs: about 0.1 %).  Batch 3..32 run on
 * the bf16 matrix cores (weights times their block scale exact in bf16 for
 * scale bytes 2..252, products exact, fp32 accumulation).  Partial sums are
 * combined in a fixed order: the same bits on every run.  silu is evaluated
 * with the hardware exp2 and reciprocal (within a few units in the last
 * place of fp32).
 */
tt_status tt_mxfp4_gateup_swiglu(const void *w_gu, int64_t inter,
                                 int64_t hidden, const void *x, int64_t batch,
                                 void *out, int32_t out_dtype, void *stream);

/*
 * Top-k routing ("ThinTensor Improvements": exact routing; MoE router stage
 * of "Dev Log #2"): per token, the topk largest bf16 logits in descending
 * order, ties to the lower expert index; w = softmax of the selected logits
 * (fp32).  logits: bf16 [batch][n_experts] (finite); ids: i32 [batch][topk];
 * w: f32 [batch][topk].  1 <= topk <= min(n_experts, TT_MAX_TOPK),
 * n_experts <= TT_MAX_EXPERTS.  Results stay on the device.
 */
tt_status tt_moe_route_topk(const void *logits, int64_t batch,
                            int64_t n_experts, int64_t topk, int32_t *ids,
                            float *w, void *stream);

/*
 * Routed-expert gate/up with SwiGLU ("numerical drift & speedups": matvec
 * over the selected experts fused with SwiGLU):
 *   h[b][j][:] = gate/up SwiGLU of expert ids[b][j] applied to x[b].
 * bank: n_experts gate/up packs back to back, each
 * tt_mxfp4_gateup_pack_bytes(inter, hidden) bytes.  ids: device i32
 * [batch][topk], read on the device (no host synchronisation).  An id
 * outside [0, n_experts) yields a NaN row and no weight read.
 * h: [batch][topk][inter] of h_dtype.
 */
tt_status tt_moe_mxfp4_gateup_swiglu(const void *bank, int64_t n_experts,
                                     int64_t inter, int64_t hidden,
                                     const void *x, int64_t batch,
                                     const int32_t *ids, int64_t topk,
                                     void *h, int32_t h_dtype, void *stream);

/*
 * Routing fused into the routed-expert gate/up: the same top-k selection and
 * softmax weights as tt_moe_route_topk (bit-identical ids and weights),
 * computed inside the gate/up kernel from the logits, followed by the same
 * gate/up SwiGLU as tt_moe_mxfp4_gateup_swiglu.  Saves one launch per layer.
 * logits: bf16 [batch][n_experts]; ids, w: outputs [batch][topk] (for the
 * down projection); h: [batch][topk][inter] of h_dtype.
 */
tt_status tt_moe_mxfp4_route_gateup_swiglu(const void *bank, int64_t n_experts,
                                           int64_t inter, int64_t hidden,
                                           const void *x, int64_t batch,
                                           const void *logits, int64_t topk,
                                           int32_t *ids, float *w, void *h,
                                           int32_t h_dtype, void *stream);

/*
 * Routed-expert down projection and weighted combine ("Dev Log #2": an MoE
 * model's expert stage after its router; "numerical drift & speedups":
 * MXFP4 matvecs over the selected experts; the gpt-oss-20b-shaped layer
 * runs gate/up SwiGLU and down per expert, weighted by the routing):
 *   y[b][r] = sum_{j = 0..topk-1} w[b][j] * ps_d[e][r] *
 *             sum_k Wd[e][r][k] * h[b][j][k],      e = ids[b][j]
 * down_bank: n_experts packs of tt_mxfp4_matrix_pack_bytes(hidden, inter).
 * h: [batch][topk][inter] of h_dtype (TT_F32 or TT_BF16); w: f32
 * [batch][topk]; y: [batch][hidden] of y_dtype.  A bad id makes the whole
 * row NaN.  No atomics: each slot's K parts are summed in order, slot j's
 * term is w_j (ps_d dot_j), and the terms are added in a fixed tree order
 * (slots j and j + 4, then quarters (0 + 1) + (2 + 3)), the same bits on
 * every run.  bf16 h
 * runs on the scaled FP4 x FP8 matrix instruction (the numerics of
 * tt_mxfp4_gateup_swiglu at batch 1), fp32 h on the vector ALUs in fp32.
 */
tt_status tt_moe_mxfp4_down_combine(const void *down_bank, int64_t n_experts,
                                    int64_t hidden, int64_t inter,
                                    const void *h, int32_t h_dtype,
                                    const int32_t *ids, const float *w,
                                    int64_t batch, int64_t topk,
                                    void *y, int32_t y_dtype, void *stream);

/*
 * Grouped affine INT4 matvec ("numerical drift & speedups": dense INT4
 * Q/K/V/O):  y[b][r] = sum_k s[r][g(k)] * (q[r][k] - z[r][g(k)]) * x[b][k].
 * w_packed from tt_pack_int4; group must be 128; k even, k <= TT_MAX_K;
 * x bf16 [batch][k]; y [batch][n] of y_dtype.  Each group's sum of
 * (128 + q) * x is taken on the bf16 matrix cores in fp32 (all operands
 * exact in bf16), then s * (sum - (128 + z) * sum x) is added in fp32.
 */
tt_status tt_int4_gemv(const void *w_packed, int64_t n, int64_t k,
                       int64_t group, const void *x, int64_t batch, void *y,
                       int32_t y_dtype, void *stream);

/*
 * Row-scaled FP8 matvec (kerbin.cskartikey.dev/@satvikhardat, "Dev Log #3 --
 * SmolLM3-3B Results": the quality FP8 profile keeps gate/up and the middle
 * down projections in FP8 and runs them as scaled matvecs -- the row's sum
 * of weight * activation in fp32, times the row scale):
 *   y[b][r] = scale[r] * sum_k w[r][k] * x[b][k]
 * w is FP8 E4M3 (OCP 8-bit floating point, the E4M3 encoding: bias 7, no
 * infinities, S.1111.111 = NaN; the pages say "FP8" only).  In this library
 * it serves the dense down projection after the gate/up SwiGLU (x = its
 * output h, fp32 or bf16).
 *
 * tt_fp8_pack_bytes / tt_pack_fp8_matrix: canonical codes u8[n][k] and
 * scale f32[n] (NULL = ones) -> the private tiled layout (8-row tiles;
 * host buffers).
 * tt_fp8_gemv: w_packed from tt_pack_fp8_matrix (device); x [batch][k] of
 * x_dtype (TT_F32 or TT_BF16), 16-byte aligned, k a multiple of 8 (bf16) or
 * 4 (fp32), k <= TT_MAX_K_FP8; y [batch][n] of y_dtype.  Products and sums
 * in fp32 (bf16 activations: on the bf16 matrix cores, every operand exact),
 * the row scale applied to the full sum.
 */
int64_t tt_fp8_pack_bytes(int64_t n, int64_t k);
tt_status tt_pack_fp8_matrix(const uint8_t *codes, const float *scale,
                             int64_t n, int64_t k, void *dst, int64_t dst_bytes);
tt_status tt_fp8_gemv(const void *w_packed, int64_t n, int64_t k, const void *x,
                      int32_t x_dtype, int64_t batch, void *y, int32_t y_dtype,
                      void *stream);

/*
 * Single-token grouped-query attention over a bf16 KV cache
 * (kerbin.cskartikey.dev/@satvikhardat, "Dev Log #3 -- SmolLM3-3B Results":
 * each query head h reads kv head g = h / (hq / hkv); scores are key . query
 * times the scale; the output is the softmax-weighted sum of the values):
 *   s_t     = scale * sum_d K[g][t][d] q[h][d],  t = 0 .. T-1
 *   out[h]  = sum_t softmax(s)_t V[g][t]
 * q: bf16 [hq][d]; k_cache, v_cache: bf16, row t of kv head g at element
 * ((g * tcap) + t) * d, T <= tcap (all device memory, 16-byte aligned);
 * d is 64 or 128; hq / hkv is 1, 2, 4 or 8; out [hq][d] of out_dtype.
 * workspace: device memory of at least tt_gqa_attention_workspace_bytes
 * bytes for the per-chunk partial results (hq x chunks x (d + 2) floats;
 * chunks of 32 positions for 256 / d * 64 < T <= 2048, of 64 otherwise); it
 * needs no initialisation, its contents are overwritten, and calls that
 * share one workspace must not overlap.  Scores are bf16 x bf16 products
 * summed in fp32, the softmax weights enter the value sum as two bf16
 * parts, exponentials and sums are fp32, and the chunks are combined in a
 * fixed order (the same bits on every run).  One kernel launch when T <=
 * 256 / d * 64 (one workgroup per kv head), two otherwise.
 */
int64_t tt_gqa_attention_workspace_bytes(int64_t hq, int64_t hkv, int64_t d, int64_t T);
tt_status tt_gqa_attention_decode(const void *q, const void *k_cache, const void *v_cache,
                                  int64_t hq, int64_t hkv, int64_t d, int64_t tcap,
                                  int64_t T, float scale, void *out, int32_t out_dtype,
                                  void *workspace, int64_t workspace_bytes, void *stream);
/*
 * tt_gqa_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under stream capture that must not
 * allocate, tight serving loops, harnesses that forbid allocation).  The
 * per-chunk partials live in one array of TT_ATTN_SCRATCH_BYTES per device
 * that the library holds from its first use on that device until the process
 * ends; the call allocates nothing.  Same arguments, kernels and results as
 * tt_gqa_attention_decode (the same bits).  TT_E_SIZE when
 * tt_gqa_attention_workspace_bytes(hq, hkv, d, T) exceeds
 * TT_ATTN_SCRATCH_BYTES (8 MiB: Phi-4-shaped heads 40 / 10 x 128 up to about
 * 25,000 positions).  Every such call on one device shares that array, so
 * calls that overlap on one device (two streams, or two host threads) race
 * and must be ordered by the caller.
 */
#define TT_ATTN_SCRATCH_BYTES (8 << 20)
tt_status tt_gqa_attention_decode_noalloc(const void *q, const void *k_cache,
                                          const void *v_cache, int64_t hq, int64_t hkv,
                                          int64_t d, int64_t tcap, int64_t T, float scale,
                                          void *out, int32_t out_dtype, void *stream);


/*
 * Decoded weights, for checking the packed layouts bit for bit (the formats
 * the calls above read: MXFP4 of "Dev Log #4", with the OCP MX v1.0 element
 * and scale encodings; affine INT4 of "Implemented a huge list of fixes";
 * FP8 of "Dev Log #3"): w[r][k] = E2M1(code) * 2^(e-127) rounded once to
 * fp32 (NaN for e = 0xFF).
 * tt_mxfp4_dequantize takes a tt_pack_mxfp4_matrix pack (w_out [n][k],
 * ps_out [n] or NULL); tt_mxfp4_gateup_dequantize takes a gate/up pack and
 * writes gate and up separately (any of the four outputs may be NULL, not
 * both matrices).  tt_int4_dequantize writes s * (q - z) in fp32 [n][k].
 */
tt_status tt_mxfp4_dequantize(const void *packed, int64_t n, int64_t k,
                              float *w_out, float *ps_out, void *stream);
tt_status tt_mxfp4_gateup_dequantize(const void *packed, int64_t inter,
                                     int64_t hidden, float *g_out,
                                     float *u_out, float *g_ps, float *u_ps,
                                     void *stream);
tt_status tt_int4_dequantize(const void *packed, int64_t n, int64_t k,
                             int64_t group, float *w_out, void *stream);
/* FP8: w_out [n][k] = E4M3(code) in fp32 (NaN for S.1111.111), scale_out
 * [n] or NULL. */
tt_status tt_fp8_dequantize(const void *packed, int64_t n, int64_t k,
                            float *w_out, float *scale_out, void *stream);

/* ---------------------------------------------------------------------- */
/* Measurement                                                             */
/* ---------------------------------------------------------------------- */

/*
 * A plain read of `bytes` bytes of device memory (16-byte aligned, a multiple
 * of 16) with 16-byte loads: 256-lane workgroups, each lane issuing
 * loads_per_lane (1, 2, 4 or 8) loads before using any.  Nothing of the
 * method is computed; it is the bandwidth ceiling a streaming kernel of the
 * same size can be compared with.  sink: 4 bytes of device memory, written
 * only when the loaded data folds to one particular word.
 */
tt_status tt_stream_read(const void *buf, int64_t bytes, int32_t loads_per_lane,
                         uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TT_H */
