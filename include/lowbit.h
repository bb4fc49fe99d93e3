/*
 * lowbit.h -- C ABI of liblowbit.so, the MI355X (gfx950) low-bit linear hot path:
 *   - a fused producer: residual += input; y = RMSNorm(residual) * weight;
 *     y quantized to FP4 E2M1 with per-block scales;
 *   - standalone FP4 quantize / dequantize of bf16 tensors;
 *   - a block-scaled A4W4 GEMM, out = epilogue(alpha * A . B^T), with BF16 or
 *     NVFP4 output.
 *
 * Sources of the operations (web pages):
 *   [FI]  FlashInfer, cute_dsl/add_rmsnorm_fp4quant.py: AddRMSNormFP4QuantKernel
 *         and add_rmsnorm_fp4quant() (operation list in the module docstring,
 *         kernel phases 1-3, API asserts and output allocation).
 *   [FRT] FlashRT fp4-gemm README: "Available Functions", "Tensor Contract",
 *         the variant list, and the "Validation" paragraph.
 *   [WOA] vLLM API docs, deepseek_v41/nvidia/ops/fused_wo_a: FusedWoAKernel
 *         (device_kernel: the activation quant stage with inverse RoPE; the
 *         MXFP8 format of its operands).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees memory, never synchronizes the device, and
 *     launches only on `stream` (NULL = the null stream).
 *   - bf16 tensors are row-major uint16 bit patterns.  Packed FP4 tensors are
 *     row-major uint8 of shape (rows, K/2): element 2j of a row sits in the low
 *     nibble of byte j, element 2j+1 in the high nibble.
 *   - Formats: LOWBIT_NVFP4 = 16-element blocks with FP8 E4M3 scales and an
 *     optional fp32 global scale gs (folded into the block scale on the way
 *     in: dequant = E2M1 * scale / gs); LOWBIT_MXFP4 = 32-element blocks with
 *     UE8M0 scales 2^(b-127) (OCP MX: e = floor(log2 amax) - 2).
 *     Rounding is to nearest, ties to the even code, saturating at 6 (E2M1)
 *     and 448 (E4M3); the sign of a value that rounds to zero is kept.
 *   - Scale layouts (per operand, `rows` x `K/B` scale bytes):
 *       LOWBIT_SF_LINEAR: row-major bytes, offset = row*(K/B) + kb.
 *       LOWBIT_SF_TILED : rows grouped by 32, blocks by 8; each group is 256
 *         bytes = 64 little-endian words; groups ordered row-group major;
 *         size ceil(rows/32)*ceil((K/B)/8)*256.  With j = kb % 8, block kb
 *         of a row is
 *           MXFP4: byte (j%2) + 2*(j/4) of word ((j/2)%2)*32 + row%32, so
 *                  word h*32 + r holds blocks {2h, 2h+1, 2h+4, 2h+5} of
 *                  row r (one word per MFMA lane feeds the four scaled-MFMA
 *                  K-steps of a 256-element superstep through the byte select);
 *           NVFP4: byte j%4 of word (j/4)*32 + row%32, so word c*32 + r
 *                  holds blocks 4c..4c+3 of row r (the four 16-blocks a lane
 *                  half dequantizes in a 128-element stage).
 *         Padding bytes are written as zero by every producer and must be
 *         zero in any TILED input.
 *       LOWBIT_SF_SWZ128: [FI]'s 128 x 4 swizzle, quantization side only
 *         (the definition is at the lowbit_sf_layout enum below).
 *   - Alignment: packed/bf16 tensor pointers 16 bytes; scale pointers 4 bytes
 *     (TILED) or 1 byte (LINEAR, SWZ128); global scales 4 bytes.
 *   - Errors are returned, never raised; on any error nothing is launched and
 *     no output is touched.  Asynchronous launch failures surface as
 *     LOWBIT_EHIP.  The device must be gfx950 (LOWBIT_EDEVICE otherwise).
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOWBIT_OK = 0,
  LOWBIT_EINVAL = 1,      /* bad enum, NULL pointer, format/argument combination */
  LOWBIT_EALIGN = 2,      /* pointer alignment */
  LOWBIT_ESHAPE = 3,      /* sizes: K % B, H < 64, rows < 0, variant invalid for the shape */
  LOWBIT_EDEVICE = 4,     /* current device is not gfx950 */
  LOWBIT_EHIP = 5,        /* a HIP runtime call or launch failed */
} lowbit_status;

/* NVFP4: 16-element blocks, E4M3 scales, optional fp32 global scale.
 * MXFP4: 32-element blocks, UE8M0 scales.  Both pack two E2M1 codes per byte:
 *        packed (rows, K/2), element 2j in the low nibble of byte j.
 * MXFP8: 32-element blocks, UE8M0 scales, E4M3 elements, one byte each:
 *        packed (rows, K) ([WOA]'s format).  Scale rule e = clamp(floor(log2
 *        amax) - 8, -127, 127) (OCP MX, emax 8 for E4M3); elements
 *        nearest-even, saturating at 448, sign kept.  LINEAR scales for the
 *        producer, quantizer, dequantizer and GEMM operands; the FP8 GEMM
 *        output (lowbit_gemm_fp8) also takes the 128 x 4 layout.
 * NVFP4_B32: the NVFP4 rule (E4M3 scales, optional global scale, clamp at
 *        448) on 32-element blocks ([FI] add_rmsnorm_fp4quant's E4M3 scale
 *        format at block size 32); packed like NVFP4.  Producer, quantizer and
 *        dequantizer only, LINEAR scales only; the GEMMs return LOWBIT_EINVAL. */
/* MXFP8_MMA: GEMM operands in the MXFP8 format (the same bytes and LINEAR
 *        scales as LOWBIT_MXFP8; quantize them with LOWBIT_MXFP8), contracted
 *        on gfx950's scaled FP8 MFMA instead of the exact bf16 path -- as
 *        [WOA]'s MMA stage runs its block-scaled MXFP8 contraction on the
 *        hardware MMA.  That instruction adds the products of a 32-element
 *        block in a narrower window than fp32: products far below the block's
 *        largest lose low bits.  Measured on the MI355X, the result differs
 *        from the exact sum by at most 2^-11.4 * sum |a_k * b_k| (random codes
 *        over the whole E4M3 range with block scales spread over 20 binades);
 *        the parity bound of this format is |out - exact| <= 2^-7 |exact| +
 *        2^-10 * sum |a_k * b_k|, against 1e-6 for the other formats.  A single
 *        product per output stays exact.  GEMM entry points only (the
 *        quantization side, lowbit_sf_bytes aside, returns LOWBIT_EINVAL);
 *        above 128 rows with K % 128 == 0 and 4-byte aligned scales it runs
 *        the same 256 x 256 schedule as the exact path, 1.3-1.8x faster on
 *        the measured prefill shapes; elsewhere (the decode shapes, other K)
 *        it runs the exact path. */
typedef enum {
  LOWBIT_NVFP4 = 0,
  LOWBIT_MXFP4 = 1,
  LOWBIT_MXFP8 = 2,
  LOWBIT_NVFP4_B32 = 3,
  LOWBIT_MXFP8_MMA = 4
} lowbit_format;
/* LOWBIT_SF_SWZ128: the 128 x 4 swizzled scale layout of [FI]'s producer
 * (its swizzled output): rows grouped by 128 and blocks by 4, each tile 512
 * contiguous bytes, tiles row-tile major with ceil(K/B/4) tiles per row tile;
 * inside a tile row r and block kb sit at byte 16*(r%32) + 4*((r%128)/32) +
 * kb%4.  lowbit_sf_bytes = ceil(rows/128) * ceil(K/B/4) * 512; padding bytes
 * are written zero.  Producer, quantizer and dequantizer with NVFP4 or MXFP4,
 * and the MXFP8 output of lowbit_gemm_fp8 ([WOA]'s F8_128x4 scale bytes);
 * GEMM operands do not take it (LOWBIT_EINVAL): lowbit_sf_convert rewrites it
 * into a layout they take. */
typedef enum { LOWBIT_SF_LINEAR = 0, LOWBIT_SF_TILED = 1, LOWBIT_SF_SWZ128 = 2 } lowbit_sf_layout;

/* GEMM schedule: -1 picks by shape (and by the workspace offered); 0 =
 * decode (weights as the MFMA row operand, K split across the waves of a
 * workgroup, for small M); 1 = prefill (LDS-staged macro tiles, for large M);
 * 2 = split-K ([FRT] "Available Functions": the stream-K down-projection
 * functions nvfp4_gemm_streamk_bf16 / _streamk_bias_bf16): K split across
 * workgroups as well, each writing fp32 partial tiles into the caller's
 * workspace, which a second kernel sums in a fixed order (the result does not
 * depend on timing) before the epilogue.  M <= 128 (decode tiles, or NVFP4's
 * 128 x 384 tiles above 64 rows), or, above 128 rows, NVFP4 with K % 64 == 0
 * on the 128 x 384 tiles and MXFP8 (exact or LOWBIT_MXFP8_MMA) with
 * K % 128 == 0 on the 256 x 256 tiles (the automatic choice: only when those
 * tiles number at most 128, i.e. fill at most half the CUs).  MXFP4 splits
 * only at M <= 128.  Cf. [FRT] `variant`. */
#define LOWBIT_VARIANT_AUTO (-1)
#define LOWBIT_VARIANT_DECODE 0
#define LOWBIT_VARIANT_PREFILL 1
#define LOWBIT_VARIANT_SPLITK 2

/* Human-readable name of a status. */
const char* lowbit_status_str(lowbit_status s);

/* Bytes of the scale buffer for a (rows, k) operand in the given format and
 * layout (cf. [FRT] sfa_size_bytes).  Returns 0 for invalid arguments. */
size_t lowbit_sf_bytes(int64_t rows, int64_t k, lowbit_format fmt, lowbit_sf_layout layout);

/* Fused add + RMSNorm + FP4 quantization ([FI] AddRMSNormFP4QuantKernel).
 * For each of the M rows of H elements:
 *   h = fl32(input + residual); residual <- bf16(h)            (in place)
 *   rstd = fl32(1 / sqrt(sum(h^2) / H + eps))   (sum of the fp32 h, in fp64)
 *   y = fl32(fl32(bf16(h) * rstd) * weight)
 *   per block: NVFP4 s = E4M3(min(fl32(fl32(gs*amax)/6), 448)),
 *              inv = fl32(fl32(1/s)*gs) (0 if s == 0), code = E2M1(fl32(y*inv));
 *              MXFP4 e = clamp(floor(log2 amax) - 2, -127, 127), byte e+127,
 *              code = E2M1(y * 2^-e).
 * input, residual: bf16 (M, H); weight: bf16 (H); out_packed: uint8 (M, H/2);
 * out_sf: lowbit_sf_bytes(M, H, fmt, layout) bytes.
 * global_scale: NVFP4 only, device fp32[1] or NULL (= 1.0); must be NULL for
 * MXFP4.  Requires H % B == 0 and H >= 64 ([FI] asserts), M >= 0 (M == 0 is
 * a no-op).  `input` must not alias `residual`. */
lowbit_status lowbit_add_rmsnorm_quant(const void* input, void* residual, const void* weight,
                                       int64_t M, int64_t H, float eps, lowbit_format fmt,
                                       lowbit_sf_layout layout, const float* global_scale,
                                       uint8_t* out_packed, uint8_t* out_sf, hipStream_t stream);

/* The same with fp16 input, residual and weight ([FI] add_rmsnorm_fp4quant
 * accepts float16 as well as bfloat16 tensors): every bf16 above reads fp16,
 * and the residual write-back rounds h to fp16 (nearest-even; |h| >= 65520
 * becomes an infinity, as an IEEE conversion does).  Same checks, layouts and
 * outputs. */
lowbit_status lowbit_add_rmsnorm_quant_fp16(const void* input, void* residual, const void* weight,
                                            int64_t M, int64_t H, float eps, lowbit_format fmt,
                                            lowbit_sf_layout layout, const float* global_scale,
                                            uint8_t* out_packed, uint8_t* out_sf, hipStream_t stream);

/* The fused producer writing its block scales in two layouts in one pass
 * ([FI] AddRMSNormFP4QuantKernel's option to emit the 128 x 4 swizzled scale
 * tensor and an unswizzled copy together).  Same arithmetic, checks and
 * outputs as lowbit_add_rmsnorm_quant with layout `layout` (LOWBIT_SF_TILED,
 * the GEMM's own layout, or LOWBIT_SF_SWZ128, the page's) into out_sf
 * (lowbit_sf_bytes(M, H, fmt, layout) bytes, padding bytes zero), and the
 * same scale bytes row-major into out_sf_linear (lowbit_sf_bytes(M, H, fmt,
 * LOWBIT_SF_LINEAR) bytes).  NVFP4 and MXFP4 only (EINVAL otherwise, and for
 * layout LOWBIT_SF_LINEAR); out_sf_linear NULL with M > 0: EINVAL.  The two
 * scale buffers must not overlap each other or the other outputs. */
lowbit_status lowbit_add_rmsnorm_quant_both_sf(const void* input, void* residual, const void* weight,
                                               int64_t M, int64_t H, float eps, lowbit_format fmt,
                                               lowbit_sf_layout layout, const float* global_scale,
                                               uint8_t* out_packed, uint8_t* out_sf, uint8_t* out_sf_linear,
                                               hipStream_t stream);

/* The same with fp16 input, residual and weight, as lowbit_add_rmsnorm_quant_fp16. */
lowbit_status lowbit_add_rmsnorm_quant_both_sf_fp16(const void* input, void* residual, const void* weight,
                                                    int64_t M, int64_t H, float eps, lowbit_format fmt,
                                                    lowbit_sf_layout layout, const float* global_scale,
                                                    uint8_t* out_packed, uint8_t* out_sf,
                                                    uint8_t* out_sf_linear, hipStream_t stream);

/* Quantize a bf16 (rows, K) tensor: the per-block rule above with y = x
 * ([FRT] quantize_fp4_sfa_bf16; used for activations and prepacked weights).
 * Requires K % B == 0, rows >= 0. */
lowbit_status lowbit_quantize(const void* x, int64_t rows, int64_t K, lowbit_format fmt,
                              lowbit_sf_layout layout, const float* global_scale,
                              uint8_t* out_packed, uint8_t* out_sf, hipStream_t stream);

/* Quantize an fp16 (rows, K) tensor: y = f32(x) (exact), then the same rule
 * ([FRT] quantize_fp4_sfa_fp16).  Same checks and outputs as lowbit_quantize. */
lowbit_status lowbit_quantize_fp16(const void* x, int64_t rows, int64_t K, lowbit_format fmt,
                                   lowbit_sf_layout layout, const float* global_scale,
                                   uint8_t* out_packed, uint8_t* out_sf, hipStream_t stream);

/* Inverse RoPE + MX quantization of attention rows ([WOA] FusedWoAKernel
 * device_kernel, its activation quant stage: the rotary part of each head
 * rotated back, 32-element blocks with an MX scale).  x: bf16 (T, heads, D),
 * row (t, h) of D elements; its last R elements (from nope = D - R on) carry
 * RoPE.  positions: int64 (T), the table row of each token; rope: fp32 (P, R),
 * each row cos[0 .. R/2) then sin[0 .. R/2).  For each pair p of the rotary
 * slice, elements k = nope + 2p and k + 1, c = rope[pos][p],
 * s = rope[pos][p + R/2]:
 *   even' = fma(even, c, fl32(odd * s)),  odd' = fma(odd, c, -fl32(even * s))
 * (the inverse rotation, the second product rounded to fp32 first).  Each
 * 32-element block of the fp32 row then takes amax' = max(amax, fl32(1e-10))
 * (the page's floor, so an all-zero block is not scale byte 0 here) and the
 * OCP MX rule on it: e = clamp(floor(log2 amax') - emax, -127, 127), byte
 * e + 127, elements encode(y * 2^-e), nearest-even and saturating with the
 * sign kept.  fmt LOWBIT_MXFP8 (the page's: E4M3 elements, emax 8, packed
 * (T*heads, D), LINEAR scales) or LOWBIT_MXFP4 (E2M1, emax 2, packed
 * (T*heads, D/2), any FP4 scale layout, for the FP4 GEMM).  out_sf:
 * lowbit_sf_bytes(T*heads, D, fmt, layout) bytes (padding written zero).
 * Requires D % 32 == 0 (32 <= D <= 32768), 0 <= R <= D with R even, P >= 1
 * when R > 0, heads >= 1, T >= 0 (T == 0 is a no-op), and T * heads * D / 8
 * below 2^31 (with the rows rounded up to 128); positions and rope may
 * be NULL when R == 0.  A position outside [0, P) reads the nearest end row
 * of the table (the table is never read outside).  Alignment: x and
 * out_packed 16 bytes, positions 8, rope 4. */
lowbit_status lowbit_rope_quant(const void* x, const int64_t* positions, const float* rope, int64_t T,
                                int64_t heads, int64_t D, int64_t R, int64_t P, lowbit_format fmt,
                                lowbit_sf_layout layout, uint8_t* out_packed, uint8_t* out_sf,
                                hipStream_t stream);

/* Dequantize to bf16: x = bf16(fl32(E2M1 * scale / gs)) (NVFP4, gs from
 * global_scale or 1.0) or bf16(E2M1 * 2^(b-127)) (MXFP4; global_scale NULL)
 * ([FRT] dequantize_fp4_sfa_fp16 with bf16 output; lowbit_dequantize_fp16
 * below gives its fp16 output). */
lowbit_status lowbit_dequantize(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K,
                                lowbit_format fmt, lowbit_sf_layout layout,
                                const float* global_scale, void* out, hipStream_t stream);

/* lowbit_dequantize with fp16 output ([FRT] dequantize_fp4_sfa_fp16): the
 * same binary32 values rounded to IEEE binary16, nearest-even (values from
 * 65520 up in magnitude become infinity; small ones fp16 subnormals or
 * zero).  out: fp16 (rows, K); arguments, checks and errors as
 * lowbit_dequantize. */
lowbit_status lowbit_dequantize_fp16(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K,
                                     lowbit_format fmt, lowbit_sf_layout layout,
                                     const float* global_scale, void* out, hipStream_t stream);

/* Scale bytes rewritten from one layout into another: for every row r < rows
 * and block kb < k/B, the byte of (r, kb) in src_layout is written at (r, kb)
 * of dst_layout; the destination's padding bytes (TILED, SWZ128) are written
 * zero, the source's are not read.  [FRT] "Tensor Contract" hands its GEMM
 * the operand scales in the 128 x 4 layout (CUTLASS SFA / SFB), which the
 * GEMMs below do not read: rewritten as TILED (FP4 formats) or LINEAR they
 * can be, once, for prepacked weights.  Likewise the 128 x 4 scales of
 * lowbit_gemm_fp8 become the LINEAR ones an MXFP8 GEMM operand takes.
 * src: lowbit_sf_bytes(rows, k, fmt, src_layout) bytes; dst:
 * lowbit_sf_bytes(rows, k, fmt, dst_layout) bytes, at most 8 GiB (ESHAPE);
 * device pointers, any alignment, the two buffers must not overlap
 * (LOWBIT_EINVAL).  Every (format, layout) pair that lowbit_sf_bytes sizes is
 * taken (TILED: NVFP4 and MXFP4 only; equal layouts copy).  Requires
 * k % B == 0, k >= B and rows >= 0 (rows == 0 is a no-op). */
lowbit_status lowbit_sf_convert(const uint8_t* src, lowbit_sf_layout src_layout, uint8_t* dst,
                                lowbit_sf_layout dst_layout, int64_t rows, int64_t k, lowbit_format fmt,
                                hipStream_t stream);

/* Block-scaled GEMM ([FRT] nvfp4_gemm_bf16 and its epilogue family).
 * a: packed (M, K/2); b: packed (N, K/2) (the weight, "B^T" row-major);
 * sfa / sfb: their scales in sfa_layout / sfb_layout; both operands use `fmt`.
 * acc[m,n] = sum_k Ahat[m,k] * Bhat[n,k] with Ahat = E2M1 * scale (no global
 * scale: pass alpha = 1/(gsA*gsB) for NVFP4 operands), accumulated in fp32.
 * MXFP8 operands ([WOA]'s format: a (M, K), b (N, K), one E4M3 byte an
 * element, LINEAR UE8M0 scales) are dequantized to bf16 -- exact while
 * E4M3 * 2^e is a normal bf16, i.e. scale bytes 10..246 -- and accumulated in
 * fp32 by the bf16 MFMA; they run the decode schedule (M <= 128), the
 * 256 x 256 prefill schedule (K % 128 == 0, 4-byte aligned scale buffers) or
 * the 64-byte-stage one (other K), and split-K.
 * out: bf16 (M, N) = bf16(alpha*acc [+ bias[n]] [+ residual[m,n]]) or
 * bf16(GELU(alpha*acc + bias[n])), GELU(t) = 0.5 t (1 + erf(t/sqrt 2)).
 * bias: bf16 (N); residual: bf16 (M, N) (may alias out).
 * Requires K % B == 0, K >= B, M, N >= 0 (empty is a no-op).
 * variant: LOWBIT_VARIANT_*; an explicit variant that cannot run the shape
 * returns LOWBIT_ESHAPE instead of silently picking another schedule.
 * NVFP4 with K % 32 == 16 (packed rows of 8 mod 16 bytes) runs on the decode
 * schedules only, at any M (more than 128 rows go as consecutive launches
 * over 128-row slices); LOWBIT_VARIANT_PREFILL returns LOWBIT_ESHAPE for it.
 * workspace, workspace_bytes: device scratch for the split-K partials
 * (16-byte aligned), owned by the caller; NULL / 0 = none.  With
 * LOWBIT_VARIANT_AUTO the split-K schedule runs only when it is offered at
 * least lowbit_gemm_workspace_bytes(M, N, K, fmt, LOWBIT_VARIANT_AUTO) bytes
 * (and that is non-zero); LOWBIT_VARIANT_SPLITK needs
 * lowbit_gemm_workspace_bytes(M, N, K, fmt, LOWBIT_VARIANT_SPLITK) bytes
 * (LOWBIT_EINVAL with less) and a shape it can split (LOWBIT_ESHAPE
 * otherwise: K of two supersteps at least; above 128 rows NVFP4 with
 * K % 64 == 0 or MXFP8 with K % 128 == 0); above 64 NVFP4 rows or 128
 * MXFP8 ones, LINEAR scale buffers 4-byte aligned (LOWBIT_EALIGN; the
 * automatic choice then runs unsplit).  The workspace contents need no initialisation
 * and are left undefined; two launches in flight on different streams must
 * not share one. */
lowbit_status lowbit_gemm_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                               const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                               lowbit_format fmt, lowbit_sf_layout sfa_layout,
                               lowbit_sf_layout sfb_layout, float alpha, void* out, int variant,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
lowbit_status lowbit_gemm_bias_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                    const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                    lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                    lowbit_sf_layout sfb_layout, float alpha, const void* bias,
                                    void* out, int variant, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);
lowbit_status lowbit_gemm_residual_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                        const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                        lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                        lowbit_sf_layout sfb_layout, float alpha,
                                        const void* residual, void* out, int variant,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);
lowbit_status lowbit_gemm_bias_residual_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                             const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                             lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                             lowbit_sf_layout sfb_layout, float alpha,
                                             const void* bias, const void* residual, void* out,
                                             int variant, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);
lowbit_status lowbit_gemm_bias_gelu_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                         const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                         lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                         lowbit_sf_layout sfb_layout, float alpha,
                                         const void* bias, void* out, int variant,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* GEMM + bias + GELU emitting NVFP4 for the next projection ([FRT]
 * nvfp4_gemm_bias_gelu_nvfp4: packed FP4 plus scales, no bf16 tensor in
 * between).  y = fl32(GELU(alpha*acc + bias[n])) is quantized along N in
 * 16-blocks with E4M3 scales and global scale out_global_scale (device
 * fp32[1] or NULL = 1.0).  out_packed: uint8 (M, N/2); out_sf:
 * lowbit_sf_bytes(M, N, LOWBIT_NVFP4, out_layout) bytes.  Requires N % 16 == 0.
 * Operands NVFP4 or MXFP4 (the page's function takes FP4 operands); MXFP8
 * operands return LOWBIT_EINVAL. */
lowbit_status lowbit_gemm_bias_gelu_fp4(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                        const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                        lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                        lowbit_sf_layout sfb_layout, float alpha,
                                        const void* bias, const float* out_global_scale,
                                        uint8_t* out_packed, uint8_t* out_sf,
                                        lowbit_sf_layout out_layout, int variant,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* lowbit_gemm_bf16 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same GEMM and arguments, without a workspace: split-K partials go to a
 * static device array of LOWBIT_STATIC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends; the call allocates
 * nothing.  The array is shared by every call on a device and keeps the last
 * call's contents (the split-K partials need no initialisation), so calls
 * that overlap on one device -- on different streams, or from other
 * threads -- race on it and must be serialised by the caller.  The automatic
 * choice splits K only when its plan fits the array; LOWBIT_VARIANT_SPLITK
 * whose plan needs more (lowbit_gemm_workspace_bytes(M, N, K, fmt,
 * LOWBIT_VARIANT_SPLITK) > LOWBIT_STATIC_SCRATCH_BYTES) returns
 * LOWBIT_ESHAPE.  The first call on a device looks the array's address up
 * there (LOWBIT_EHIP if that fails); every other check is lowbit_gemm_bf16's. */
#define LOWBIT_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
lowbit_status lowbit_gemm_bf16_noalloc(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                       const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                       lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                       lowbit_sf_layout sfb_layout, float alpha, void* out,
                                       int variant, hipStream_t stream);

/* GEMM with FP8 output ([WOA] FusedWoAKernel.device_kernel output epilogue:
 * the reduced sum rounded to bf16, a 32-column block maximum, an MX scale,
 * FP8 elements).  value = bf16(alpha * acc), then each 32-run of an output row
 * is quantized as MXFP8 (the rule above; an all-zero block gets scale byte 0)
 * into out_packed: uint8 (M, N), one E4M3 byte an element, and out_sf:
 * lowbit_sf_bytes(M, N, LOWBIT_MXFP8, out_layout) bytes, out_layout
 * LOWBIT_SF_LINEAR or LOWBIT_SF_SWZ128 (the page's 128 x 4 scale bytes,
 * padding written zero).  Operands in any GEMM format; requires N % 32 == 0;
 * out_packed 16-byte aligned.  Other arguments as lowbit_gemm_bf16. */
lowbit_status lowbit_gemm_fp8(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                              const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                              lowbit_format fmt, lowbit_sf_layout sfa_layout,
                              lowbit_sf_layout sfb_layout, float alpha, uint8_t* out_packed,
                              uint8_t* out_sf, lowbit_sf_layout out_layout, int variant,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Which schedule a GEMM call with these sizes and this much workspace would
 * run (-1 auto resolved), or -1 if the sizes or the variant are invalid.
 * Host-only, launches nothing. */
int lowbit_gemm_pick_variant(int64_t M, int64_t N, int64_t K, lowbit_format fmt, int variant,
                             size_t workspace_bytes);

/* Workspace bytes the split-K schedule needs for these sizes: variant
 * LOWBIT_VARIANT_AUTO gives the amount that lets the automatic choice split
 * K (0 when it would not split: K too short for the tile count, more than
 * 128 rows in MXFP4, or more than 128 prefill tiles -- 128 x 384 for NVFP4,
 * 256 x 256 for MXFP8),
 * LOWBIT_VARIANT_SPLITK the amount an explicit split-K call needs (0 when it
 * cannot run); 0 for every other variant and for invalid sizes (cf. [FRT]
 * sfa_size_bytes, a size query beside the kernels).  Host-only. */
size_t lowbit_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, lowbit_format fmt, int variant);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
