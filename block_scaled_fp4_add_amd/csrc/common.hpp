// common.hpp -- device-side building blocks of liblowbit (gfx950 only).
//
// Element formats (FP4 E2M1, FP8 E4M3 "FN", UE8M0), the two scale layouts,
// and wave-level helpers.  Everything here is written for CDNA4: wave64,
// the hardware FP4 packing conversion and bf16 conversion of gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

constexpr int kWave = 64;

// kNV32 (the NVFP4 rule on 32-blocks): quantization only, no GEMM
enum Fmt : int { kNVFP4 = 0, kMXFP4 = 1, kMXFP8 = 2, kNV32 = 3 };
// kMXFP8Mma: MXFP8 operands (kMXFP8's bytes and scales) contracted on the
// scaled FP8 MFMA -- a GEMM format id only; its kernels run as kMXFP8 with
// GemmArgs::f8mma set
constexpr int kMXFP8Mma = 4;
// kSwz128: the producer page's 128 x 4 swizzled layout (quantization side only)
enum Layout : int { kLinear = 0, kTiled = 1, kSwz128 = 2 };
enum Epi : int { kEpiNone = 0, kEpiBias = 1, kEpiResidual = 2, kEpiBiasResidual = 3, kEpiBiasGelu = 4,
                 kEpiBiasGeluFp4 = 5, kEpiFp8 = 6 };

template <int FMT> struct FmtTraits;
template <> struct FmtTraits<kNVFP4> { static constexpr int B = 16; };
template <> struct FmtTraits<kMXFP4> { static constexpr int B = 32; };
template <> struct FmtTraits<kMXFP8> { static constexpr int B = 32; };
template <> struct FmtTraits<kNV32> { static constexpr int B = 32; };

// block scale E4M3 with the global scale folded in (NVFP4 and its 32-block form)
constexpr bool e4m3_scaled(int f) { return f == kNVFP4 || f == kNV32; }

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
// Two fp32 -> two bf16 in one 32-bit word (lo in the low half), one
// v_cvt_pk_bf16_f32 for both (the same rounding as f32_to_bf16; converting
// them one by one costs four instructions).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// IEEE binary16 (fp16), the producer's other input format: widening is exact
// (v_cvt_f32_f16); narrowing rounds to nearest-even (v_cvt_pk_f16_f32).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
// The two 16-bit halves of a word of the input format (F16: fp16, else bf16).
template <bool F16> __device__ __forceinline__ float in_lo(uint32_t w) { return F16 ? f16_lo(w) : bf16_lo(w); }
template <bool F16> __device__ __forceinline__ float in_hi(uint32_t w) { return F16 ? f16_hi(w) : bf16_hi(w); }
template <bool F16> __device__ __forceinline__ uint32_t pack_in2(float lo, float hi) {
  return F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// ---------------------------------------------------------------------------
// FP4 E2M1: two fp32 -> one byte (first value in the low nibble).  The gfx950
// conversion rounds to nearest-even, saturates at +-6 and keeps the sign of a
// value that rounds to zero; it is applied with a unit scale so that the
// quantizer's own product v = fl32(y * inv) is what gets rounded.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1x2(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}
// Eight fp32 -> 32 bits (element i in nibble i).
__device__ __forceinline__ uint32_t e2m1x8(const float* v) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
  return r;
}

// E2M1 code -> value (sign bit 3): exponent field e (bias 1), mantissa bit m;
// normal values are (2 + m) * 2^(e-2), the subnormal one is 0.5 * m.
__device__ __forceinline__ float e2m1_to_f32(uint32_t code) {
  uint32_t e = (code >> 1) & 3, m = code & 1;
  float mag = (e == 0) ? 0.5f * (float)m : (float)(2 + m) * __uint_as_float((uint32_t)(125 + e) << 23);
  return (code & 8) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// FP8 E4M3 "FN" (bias 7, max 448, no infinities): encode non-negative finite
// x with round-to-nearest-even and saturation at 448.  With e = max(floor(
// log2 x), -6) the grid step there is 2^(e-3); q = rint(x / step) counts
// steps, and code = (e + 7) * 8 + q - 8 is right both for normals (q in
// [8, 16], q == 16 carrying into the exponent) and for subnormals (e = -6).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float x) {
  if (!(x < 448.0f)) return 0x7Eu;
  int eb = (int)((__float_as_uint(x) >> 23) & 0xFF);
  int e = eb - 127;
  if (e < -6) e = -6;
  float inv_step = __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // 2^(3-e), exact
  float q = __builtin_rintf(x * inv_step);                           // exact scaling, RNE
  int code = (e + 7) * 8 + (int)q - 8;
  return code > 0x7E ? 0x7Eu : (uint32_t)code;
}
// E4M3 element (MXFP8): nearest-even, saturating at 448, the sign bit copied
// from v (so a negative value that rounds to zero gives 0x80).
__device__ __forceinline__ uint32_t e4m3_encode_signed(float v) {
  return ((__float_as_uint(v) >> 24) & 0x80u) | e4m3_encode_nonneg(fabsf(v));
}
// Eight fp32 -> eight E4M3 bytes (element i in byte i): each value clamped to
// [-448, 448] (v_med3, keeps the sign of zero), then gfx950's packed FP8
// conversion at unit scale, which rounds to nearest-even and keeps the sign
// of a value that rounds to zero (checked on the device against the
// nearest-even encoder above for every bf16 value up to 510 in magnitude).
typedef short s16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  s16x2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                                               __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f), 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f),
                                               __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f), 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint2 e4m3x8(const float* v) {
  uint2 r;
  r.x = e4m3x4(v[0], v[1], v[2], v[3]);
  r.y = e4m3x4(v[4], v[5], v[6], v[7]);
  return r;
}
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15, m = b & 7;
  float v = (e == 0) ? (float)m * 0x1p-9f : (float)(8 + m) * __uint_as_float((e + 117u) << 23);
  return (b & 0x80) ? -v : v;
}
// UE8M0 byte -> 2^(b-127) for b in [1, 254]; b == 0 gives 2^-127 (subnormal).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) {
  return b == 0 ? 0x1p-127f : __uint_as_float(b << 23);
}

// ---------------------------------------------------------------------------
// Scale layouts.  LINEAR: row * nblk + kb.  TILED: 32-row x 8-block groups of
// 256 bytes, row-group major; inside a group one 32-bit word per (lane half,
// row) holds the four blocks that lane half of a GEMM wave reads (gemm.hip),
// with j = kb % 8:
//   MXFP4: word ((j/2)%2)*32 + row%32, byte (j%2) + 2(j/4)  -- blocks
//          {2h, 2h+1, 2h+4, 2h+5}, one per quarter of a 256-element superstep;
//   NVFP4: word (j/4)*32 + row%32, byte j%4  -- blocks 4c..4c+3, the lane
//          half's blocks of a 128-element stage.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t sf_offset(int fmt, int layout, int64_t row, int64_t kb, int64_t nblk) {
  if (layout == kLinear) return row * nblk + kb;
  if (layout == kSwz128) {
    // 128-row x 4-block tiles of 512 bytes, row-tile major; inside a tile row
    // r, block kb at 16 (r % 32) + 4 ((r % 128) / 32) + kb % 4
    const int64_t tile = (row >> 7) * ((nblk + 3) >> 2) + (kb >> 2);
    return (tile << 9) + ((row & 31) << 4) + (((row >> 5) & 3) << 2) + (kb & 3);
  }
  int64_t ktiles = (nblk + 7) >> 3;
  int64_t j = kb & 7;
  int64_t base = ((row >> 5) * ktiles + (kb >> 3)) << 8;
  if (fmt == kNVFP4) return base + ((((j >> 2) << 5) + (row & 31)) << 2) + (j & 3);
  return base + (((((j >> 1) & 1) << 5) + (row & 31)) << 2) + (j & 1) + ((j >> 2) << 1);
}
__host__ __device__ inline int64_t sf_bytes_of(int layout, int64_t rows, int64_t nblk) {
  if (layout == kLinear) return rows * nblk;
  if (layout == kSwz128) return ((rows + 127) / 128) * ((nblk + 3) / 4) * 512;
  return ((rows + 31) / 32) * ((nblk + 7) / 8) * 256;
}
// blocks per row and rows the padded layouts cover (padding bytes are zero)
__host__ __device__ inline int64_t sf_pad_blocks(int layout, int64_t nblk) {
  return layout == kTiled ? (nblk + 7) / 8 * 8 : layout == kSwz128 ? (nblk + 3) / 4 * 4 : nblk;
}
__host__ __device__ inline int64_t sf_pad_rows(int layout, int64_t rows) {
  return layout == kTiled ? (rows + 31) / 32 * 32 : layout == kSwz128 ? (rows + 127) / 128 * 128 : rows;
}

// ---------------------------------------------------------------------------
// Wave reductions (wave64, butterfly over all lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// GELU, exact (erf) form, fp32, written as gelu(z) = z/2 * erfc(-z/sqrt(2))
// so that the negative tail keeps its relative precision (1 + erf cancels
// there).  erfc(x) for x >= 0 takes the published Chebyshev-fitted form of
// the "erfcc" routine in Press et al., Numerical Recipes (section 6.2):
// t * exp(-x^2 + g(t)), t = 1 / (1 + x/2), g a degree-9 polynomial in t.  Its
// coefficients here are our own least-squares refit of ln(erfc(x) e^{x^2} / t)
// over t in (0, 1] (relative error of that erfc below 1.1e-7 for x >= 0);
// erfc(-x) = 2 - erfc(x).  -x^2 is formed as fma(-z/2, z, g): z/2 is exact,
// so the exponent argument is rounded once.  Branch-free.  The fp32
// evaluation is less accurate than the fit: the roundings of the exponent
// argument (|arg| up to about 40) dominate, and with v_rcp_f32 and
// v_exp_f32 each allowed one ulp the result's relative error stays below
// 2.6e-6 for z >= -6 and 4.5e-6 for z >= -9 (operation sequence replayed on
// the CPU against a binary64 erfc).  Below -9 |gelu(z)| < 1.1e-18.
constexpr float kGeluErfcPoly[10] = {-1.26551222f, 1.00002284f, 0.37412141f,  0.09641923f, -0.18410964f,
                                     0.27173793f,  -1.12172492f, 1.4738528f, -0.81363612f, 0.1688286f};
__device__ __forceinline__ float gelu_erf(float z) {
  const float x = fabsf(z) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, x, 1.0f));
  float g = kGeluErfcPoly[9];
#pragma unroll
  for (int k = 8; k >= 0; k--) g = fmaf(g, t, kGeluErfcPoly[k]);
  const float arg = fmaf(-0.5f * z, z, g);
  const float e = t * __builtin_amdgcn_exp2f(arg * 1.44269504088896340736f);
  const float f = (z >= 0.0f) ? 2.0f - e : e;
  return 0.5f * z * f;
}

// NVFP4 block scale from a block amax (E4M3 byte and the fp32 inverse used
// to scale the block's values), global scale gs folded in:
//   s = E4M3(min(fl32(fl32(gs * amax) / 6), 448)), inv = s ? fl32(fl32(1/s) * gs) : 0
__device__ __forceinline__ uint32_t nv_block_scale(float amax, float gs, float* inv) {
  float t = __fmul_rn(gs, amax);
  float s_pre = fminf(__fdiv_rn(t, 6.0f), 448.0f);
  uint32_t sb = e4m3_encode_nonneg(s_pre);
  float sdec = e4m3_to_f32(sb);
  *inv = (sdec == 0.0f) ? 0.0f : __fmul_rn(__fdiv_rn(1.0f, sdec), gs);
  return sb;
}
// MX block scale (OCP MX): e = clamp(floor(log2 amax) - EMAX, -127, 127) with
// EMAX the element format's largest exponent (2 for E2M1, 8 for E4M3);
// returns the byte e + 127 and the exact power of two 2^-e.
template <int EMAX>
__device__ __forceinline__ uint32_t mx_block_scale_e(float amax, float* inv) {
  int eb = (int)((__float_as_uint(amax) >> 23) & 0xFF);  // amax >= 0, finite
  int sb = eb - EMAX;
  if (sb < 0) sb = 0;                                     // e = -127 (also amax == 0 / subnormal)
  *inv = __uint_as_float((uint32_t)(254 - sb) << 23);     // 2^(127 - sb) = 2^-e
  return (uint32_t)sb;
}
__device__ __forceinline__ uint32_t mx_block_scale(float amax, float* inv) { return mx_block_scale_e<2>(amax, inv); }

}  // namespace lowbit
