/*
 * lowbit_oracle.c -- plain, slow CPU oracle for the block-scaled FP4 hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no source, header, table or helper
 * with the HIP kernels.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (no FMA contraction, IEEE binary32/binary64 with subnormals).
 *
 * What it computes, and where each step comes from:
 *   - The fused producer follows the FlashInfer page "cute_dsl/add_rmsnorm_fp4quant.py",
 *     AddRMSNormFP4QuantKernel.kernel, phases 1-3 (add + residual write-back,
 *     sum of squares / rstd, per-block scale, FP4 quantize-and-pack), with the
 *     readings listed under each function below.
 *   - The inverse-RoPE + MX quantizer follows the vLLM page
 *     "deepseek_v41/nvidia/ops/fused_wo_a", FusedWoAKernel.device_kernel,
 *     its activation quant stage (inverse RoPE on the rope slice, a 32-element
 *     block maximum floored at 1e-10, an MX scale, FP8 elements).
 *   - The FP4 GEMM follows the FlashRT "fp4-gemm" README: "Tensor Contract"
 *     (A (M,K/2), B (N,K/2) packed, out (M,N) = alpha * A . B^T) and its
 *     "Validation" paragraph (dequantize exactly the bytes the kernel used,
 *     then a high-precision matmul of the dequantized low-bit values).
 *   - Element formats are written from their definitions: FP4 E2M1 (max 6),
 *     FP8 E4M3 "FN" (bias 7, max 448, no infinities), UE8M0 (2^(b-127)), as
 *     the FlashInfer page's constants FLOAT4_E2M1_MAX = 6 and
 *     FLOAT8_E4M3_MAX = 448 state; rounding is round-to-nearest, ties to the
 *     even code, saturating at the format maximum.
 *
 * Every function is a direct transcription of the definition, not a faster
 * equivalent: encoders scan the value grid, the GEMM is a triple loop in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_NVFP4 = 0, ORC_MXFP4 = 1, ORC_MXFP8 = 2, ORC_NVFP4_B32 = 3 };
enum { ORC_SF_LINEAR = 0, ORC_SF_TILED = 1, ORC_SF_SWZ128 = 2 };
enum { ORC_EPI_NONE = 0, ORC_EPI_BIAS = 1, ORC_EPI_RESIDUAL = 2, ORC_EPI_BIAS_RESIDUAL = 3,
       ORC_EPI_BIAS_GELU = 4 };

/* ------------------------------------------------------------------------- */
/* bf16 <-> fp32                                                              */
/* ------------------------------------------------------------------------- */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the upper half of a binary32; widening is exact. */
float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* Round a binary32 to bf16, nearest-even, written as "pick the nearer of the
 * two truncation neighbours" (inputs here are always finite). */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u = f32_bits(f);
    uint16_t lo = (uint16_t)(u >> 16);          /* truncation toward zero */
    uint32_t rest = u & 0xFFFFu;                /* discarded low half */
    if (rest > 0x8000u) return (uint16_t)(lo + 1);
    if (rest < 0x8000u) return lo;
    return (lo & 1u) ? (uint16_t)(lo + 1) : lo; /* exact tie: keep the even one */
}

/* ------------------------------------------------------------------------- */
/* fp16 (IEEE binary16) <-> fp32                                              */
/* ------------------------------------------------------------------------- */

/* binary16: a sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent
 * field 0 holds the subnormals f * 2^-24, field 31 infinities and NaNs.
 * Widening is exact. */
float orc_f16_to_f32(uint16_t b) {
    int sgn = b >> 15, e = (b >> 10) & 31, f = b & 1023;
    double v;
    if (e == 31) v = f ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)f, -24);
    else v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return (float)(sgn ? -v : v);
}

/* Round a binary32 to binary16, nearest-even: count the value in steps of the
 * binary16 grid of its binade (2^(E-10) for a normal value in [2^E, 2^(E+1)),
 * 2^-24 below 2^-14) and round the count to the nearest integer, ties to even
 * (rint in the default rounding mode).  A count that reaches the next binade
 * carries into the exponent.  Magnitudes from 65520, the midpoint between the
 * largest finite value 65504 and 2^16, become infinity. */
uint16_t orc_f32_to_f16(float f) {
    uint16_t sign = (f32_bits(f) >> 31) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)f);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    int e2;
    frexp(a, &e2);               /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;              /* floor(log2 a) */
    if (a == 0.0 || E < -14) {
        double q = rint(a * 0x1p24);   /* exact scaling; q <= 1024 (1024 = 2^-14) */
        return (uint16_t)(sign | (uint16_t)q);
    }
    double q = rint(ldexp(a, 10 - E));  /* in [1024, 2048] */
    if (q == 2048.0) { q = 1024.0; E += 1; }
    return (uint16_t)(sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024)));
}

/* The 16-bit input formats of the producer and the quantizer. */
enum { ORC_IN_BF16 = 0, ORC_IN_F16 = 1 };
typedef float (*orc_widen_fn)(uint16_t);
typedef uint16_t (*orc_narrow_fn)(float);
static orc_widen_fn widen_of(int dtype) { return dtype == ORC_IN_F16 ? orc_f16_to_f32 : orc_bf16_to_f32; }
static orc_narrow_fn narrow_of(int dtype) { return dtype == ORC_IN_F16 ? orc_f32_to_f16 : orc_f32_to_bf16; }

/* ------------------------------------------------------------------------- */
/* FP4 E2M1                                                                   */
/* ------------------------------------------------------------------------- */

/* Magnitudes of codes 0..7: exponent bias 1, one mantissa bit, code 1 is the
 * subnormal 0.5.  Bit 3 is the sign. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(uint8_t code) {
    double m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* Nearest E2M1 magnitude to |v|, ties to the code with mantissa bit 0 (the
 * even code), saturating at 6.  The sign of v is kept, so -0.1 gives 0x8. */
uint8_t orc_e2m1_encode(float v) {
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0) return (uint8_t)(sign | 7);
    /* a lies in [E2M1_MAG[c], E2M1_MAG[c+1]) for exactly one c in 0..6 */
    int c = 0;
    while (!(a < E2M1_MAG[c + 1])) c++;
    double mid = 0.5 * (E2M1_MAG[c] + E2M1_MAG[c + 1]); /* exact in binary64 */
    int code;
    if (a < mid) code = c;
    else if (a > mid) code = c + 1;
    else code = (c % 2 == 0) ? c : c + 1;
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------- */
/* FP8 E4M3 (OCP "FN": bias 7, no infinities, S.1111.111 is NaN, max 448)      */
/* ------------------------------------------------------------------------- */

double orc_e4m3_value(uint8_t b) {
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);      /* subnormal: 0.mmm * 2^-6 */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 value, ties to the even code, saturating at 448.  Scans the
 * 127 non-negative finite codes in increasing order. */
uint8_t orc_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int c = 0;                                   /* codes 0x00..0x7E increase */
    while (!(a < orc_e4m3_value((uint8_t)(c + 1)))) c++;
    double lo = orc_e4m3_value((uint8_t)c), hi = orc_e4m3_value((uint8_t)(c + 1));
    double mid = 0.5 * (lo + hi);               /* exact: few significant bits */
    int code;
    if (a < mid) code = c;
    else if (a > mid) code = c + 1;
    else code = (c % 2 == 0) ? c : c + 1;
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------- */
/* UE8M0: byte b encodes 2^(b-127); 255 is NaN and is never produced           */
/* ------------------------------------------------------------------------- */

double orc_ue8m0_value(uint8_t b) {
    if (b == 255) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------------------------- */
/* Scale-factor layouts                                                       */
/* ------------------------------------------------------------------------- */
/*
 * LINEAR: row-major (rows, K/B) bytes, the FlashInfer page's unswizzled
 *         layout mS[row, sf_idx].
 * TILED:  rows are grouped by 32 and scale blocks by 8.  Each 32 x 8 group is
 *         256 contiguous bytes laid out as 64 little-endian 32-bit words;
 *         groups are ordered row-group major; padding bytes are zero.  Which
 *         word and byte block kb of a row takes (j = kb % 8) depends on the
 *         format, so that one word holds the four blocks one GEMM lane reads:
 *           MXFP4: word ((j / 2) % 2) * 32 + row % 32, byte (j % 2) + 2 * (j / 4)
 *                  (word h*32 + r holds blocks {2h, 2h+1, 2h+4, 2h+5} of row r);
 *           NVFP4: word (j / 4) * 32 + row % 32, byte j % 4
 *                  (word c*32 + r holds blocks 4c .. 4c+3 of row r).
 * SWZ128: the FlashInfer page's swizzled layout (its output_swizzled path):
 *         rows grouped by 128 and blocks by 4, each 128 x 4 tile 512
 *         contiguous bytes, tiles ordered row-tile major (ceil(nblk/4) tiles
 *         per row tile).  Inside a tile, row r and block kb sit at byte
 *         16 * (r % 32) + 4 * ((r % 128) / 32) + kb % 4.  The page allocates
 *         the buffer uninitialised; here the padding bytes are zero.
 */
static int64_t block_of(int fmt) { return fmt == ORC_NVFP4 ? 16 : 32; }

/* The formats whose block scale is E4M3 with the global scale folded in:
 * NVFP4, and the same rule on 32-element blocks. */
static int e4m3_scaled(int fmt) { return fmt == ORC_NVFP4 || fmt == ORC_NVFP4_B32; }

int64_t orc_sf_bytes(int64_t rows, int64_t k, int fmt, int layout) {
    int64_t nblk = k / block_of(fmt);
    if (layout == ORC_SF_LINEAR) return rows * nblk;
    if (layout == ORC_SF_SWZ128) return ((rows + 127) / 128) * ((nblk + 3) / 4) * 512;
    return ((rows + 31) / 32) * ((nblk + 7) / 8) * 256;
}

int64_t orc_sf_offset(int64_t row, int64_t kb, int64_t nblk, int fmt, int layout) {
    if (layout == ORC_SF_LINEAR) return row * nblk + kb;
    if (layout == ORC_SF_SWZ128) {
        int64_t tile = (row / 128) * ((nblk + 3) / 4) + kb / 4;
        return tile * 512 + (row % 32) * 16 + ((row % 128) / 32) * 4 + kb % 4;
    }
    int64_t ktiles = (nblk + 7) / 8;
    int64_t tile = (row / 32) * ktiles + kb / 8;
    int64_t j = kb % 8;
    if (fmt == ORC_NVFP4) return tile * 256 + ((j / 4) * 32 + row % 32) * 4 + j % 4;
    return tile * 256 + (((j / 2) % 2) * 32 + row % 32) * 4 + (j % 2) + 2 * (j / 4);
}

/* The scale bytes of a (rows, k) operand moved from one layout to another:
 * the byte of each (row, block) goes to the same (row, block) of the
 * destination, whose padding is zero.  The FlashRT page's GEMM takes its
 * operand scales in the 128 x 4 layout (its "Tensor Contract"); this is the
 * definition the library's relayout is checked against. */
void orc_sf_convert(const uint8_t* src, int src_layout, uint8_t* dst, int dst_layout, int64_t rows,
                    int64_t k, int fmt) {
    int64_t nblk = k / block_of(fmt);
    memset(dst, 0, (size_t)orc_sf_bytes(rows, k, fmt, dst_layout));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t kb = 0; kb < nblk; ++kb)
            dst[orc_sf_offset(r, kb, nblk, fmt, dst_layout)] = src[orc_sf_offset(r, kb, nblk, fmt, src_layout)];
}

/* ------------------------------------------------------------------------- */
/* One quantization block (FlashInfer page, kernel Phase 3)                    */
/* ------------------------------------------------------------------------- */
/*
 * Input: the block's fp32 values y[0..B).  Output: the scale byte, the codes,
 * and (optional) the pre-rounding values the parity checker needs.
 *
 * NVFP4 (B = 16, E4M3 scale, global scale gs folded into the block scale --
 * the page's code multiplies gs into the scale and "not applied to input"):
 *     s_pre = min(fl32(fl32(gs * amax) / 6), 448);  sbyte = E4M3(s_pre)
 *     inv   = sdec == 0 ? 0 : fl32(fl32(1 / sdec) * gs)
 *     v_i   = fl32(y_i * inv);  code_i = E2M1(v_i)
 * NVFP4 with 32-element blocks (the page's producer takes an E4M3 scale
 * format override at block size 32): the NVFP4 rule above, amax over 32.
 * MXFP4 (B = 32, UE8M0 scale, OCP MX rule, gs unused):
 *     e = clamp(floor(log2 amax) - 2, -127, 127)  (amax == 0 gives -127)
 *     sbyte = e + 127;  v_i = y_i * 2^-e (exact);  code_i = E2M1(v_i)
 * MXFP8 (B = 32, UE8M0 scale, E4M3 elements, the same OCP MX rule with the
 * element format's largest exponent, 8 for E4M3):
 *     e = clamp(floor(log2 amax) - 8, -127, 127);  sbyte = e + 127
 *     v_i = y_i * 2^-e;  code_i = E4M3(v_i) (nearest-even, saturating at 448,
 *     sign kept), one byte per element
 */
static void quant_block(const float* y, int B, int fmt, float gs, uint8_t* codes, uint8_t* sbyte,
                        float* amax_out, float* spre_out, float* v_out) {
    float amax = 0.0f;
    for (int i = 0; i < B; i++) {
        float a = fabsf(y[i]);
        if (a > amax) amax = a;
    }
    if (amax_out) *amax_out = amax;
    if (e4m3_scaled(fmt)) {
        volatile float t = gs * amax;            /* fl32(gs * amax) */
        volatile float s_pre = t / 6.0f;         /* fl32(. / 6) */
        float sp = s_pre;
        if (sp > 448.0f) sp = 448.0f;
        if (spre_out) *spre_out = sp;
        uint8_t sb = orc_e4m3_encode(sp);
        *sbyte = sb;
        float sdec = (float)orc_e4m3_value(sb);  /* exact in fp32 */
        float inv;
        if (sdec == 0.0f) {
            inv = 0.0f;
        } else {
            volatile float r = 1.0f / sdec;      /* fl32(1 / sdec) */
            inv = r * gs;                        /* fl32(. * gs) */
        }
        for (int i = 0; i < B; i++) {
            volatile float v = y[i] * inv;
            if (v_out) v_out[i] = v;
            codes[i] = orc_e2m1_encode(v);
        }
    } else {
        const int emax = (fmt == ORC_MXFP8) ? 8 : 2;   /* largest exponent of E4M3 / E2M1 */
        int e;
        if (amax == 0.0f) {
            e = -127;
        } else {
            int E;
            (void)frexp((double)amax, &E);       /* amax = f * 2^E, f in [0.5, 1) */
            e = (E - 1) - emax;                  /* floor(log2 amax) - emax */
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        if (spre_out) *spre_out = amax;          /* the value whose binade decides e */
        *sbyte = (uint8_t)(e + 127);
        for (int i = 0; i < B; i++) {
            float v = ldexpf(y[i], -e);          /* exact unless it underflows */
            if (v_out) v_out[i] = v;
            codes[i] = (fmt == ORC_MXFP8) ? orc_e4m3_encode(v) : orc_e2m1_encode(v);
        }
    }
}

/* Re-encode a block from a given scale byte (used by the parity checker when
 * the device's scale byte differs inside the tolerance window).  v_out
 * (optional) receives the pre-rounding values. */
void orc_encode_with_scale(const float* y, int B, int fmt, float gs, uint8_t sbyte, uint8_t* codes,
                           float* v_out) {
    if (e4m3_scaled(fmt)) {
        float sdec = (float)orc_e4m3_value(sbyte);
        float inv;
        if (sdec == 0.0f) {
            inv = 0.0f;
        } else {
            volatile float r = 1.0f / sdec;
            inv = r * gs;
        }
        for (int i = 0; i < B; i++) {
            volatile float v = y[i] * inv;
            if (v_out) v_out[i] = v;
            codes[i] = orc_e2m1_encode(v);
        }
    } else {
        int e = (int)sbyte - 127;
        for (int i = 0; i < B; i++) {
            float v = ldexpf(y[i], -e);
            if (v_out) v_out[i] = v;
            codes[i] = (fmt == ORC_MXFP8) ? orc_e4m3_encode(v) : orc_e2m1_encode(v);
        }
    }
}

/* FP4: codes two per byte, element 2j in the low nibble, 2j+1 in the high.
 * MXFP8: one byte per element. */
static void pack_row(const uint8_t* codes, int64_t n, int fmt, uint8_t* out) {
    if (fmt == ORC_MXFP8) {
        memcpy(out, codes, (size_t)n);
        return;
    }
    for (int64_t j = 0; j < n / 2; j++)
        out[j] = (uint8_t)((codes[2 * j] & 15) | ((codes[2 * j + 1] & 15) << 4));
}

/* Bytes of one packed row of n elements. */
static int64_t row_bytes(int fmt, int64_t n) { return fmt == ORC_MXFP8 ? n : n / 2; }

/* Quantize one row of n fp32 values and write codes + scales in the layout. */
static void quant_row(const float* y, int64_t row, int64_t n, int fmt, float gs, int layout,
                      uint8_t* packed_row, uint8_t* sf, uint8_t* codes_tmp,
                      float* amax_row, float* spre_row, float* v_row) {
    int B = (int)block_of(fmt);
    int64_t nblk = n / B;
    for (int64_t b = 0; b < nblk; b++) {
        uint8_t sb;
        quant_block(y + b * B, B, fmt, gs, codes_tmp + b * B, &sb,
                    amax_row ? amax_row + b : NULL, spre_row ? spre_row + b : NULL,
                    v_row ? v_row + b * B : NULL);
        sf[orc_sf_offset(row, b, nblk, fmt, layout)] = sb;
    }
    pack_row(codes_tmp, n, fmt, packed_row);
}

static int check_common(int64_t rows, int64_t k, int fmt, int layout) {
    if (rows < 0 || k <= 0) return 1;
    if (fmt != ORC_NVFP4 && fmt != ORC_MXFP4 && fmt != ORC_MXFP8 && fmt != ORC_NVFP4_B32) return 1;
    if (layout != ORC_SF_LINEAR && layout != ORC_SF_TILED && layout != ORC_SF_SWZ128) return 1;
    /* MXFP8 and 32-block NVFP4 scales: LINEAR only */
    if ((fmt == ORC_MXFP8 || fmt == ORC_NVFP4_B32) && layout != ORC_SF_LINEAR) return 1;
    if (k % block_of(fmt) != 0) return 1;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Fused producer (FlashInfer page, AddRMSNormFP4QuantKernel)                  */
/* ------------------------------------------------------------------------- */
/*
 * For each row m (H elements; x, r, w are bf16 bit patterns, or fp16 with dtype
 * ORC_IN_F16, where every bf16 conversion below is the fp16 one):
 *  1. h_i = fl32(x_i + r_i); residual_i <- bf16(h_i)     (Phase 2, in place)
 *  2. S = sum_i h_i^2 over the fp32 h (the page squares the unrounded h),
 *     accumulated in binary64 (each h_i^2 is exact there);
 *     rstd = fl32(1 / sqrt(S / H + eps))  -- a correctly rounded reading of
 *     the page's rsqrt(mean_sq + eps)
 *  3. y_i = fl32(fl32(bf16(h_i) * rstd) * w_i)  (the page reads h back from its
 *     bf16 shared-memory copy and computes h * rstd * w)
 *  4. per block: quant_block above; scales go to out_sf in the layout.
 * gs: the global scale value (NVFP4 and its 32-block form; ignored for MXFP4 and MXFP8).
 * Optional diagnostics (NULL to skip): y (M*H fp32), v (M*H fp32),
 * amax and s_pre (M*H/B fp32 each), rstd (M fp32).
 */
int orc_add_rmsnorm_quant_dt(const uint16_t* x, uint16_t* residual, const uint16_t* w,
                             int64_t M, int64_t H, float eps, int fmt, int layout, float gs,
                             uint8_t* out_packed, uint8_t* out_sf,
                             float* diag_y, float* diag_v, float* diag_amax, float* diag_spre,
                             float* diag_rstd, int dtype) {
    if (check_common(M, H, fmt, layout)) return 1;
    if (dtype != ORC_IN_BF16 && dtype != ORC_IN_F16) return 1;
    const orc_widen_fn wid = widen_of(dtype);
    const orc_narrow_fn nar = narrow_of(dtype);
    int64_t B = block_of(fmt), nblk = H / B;
    memset(out_sf, 0, (size_t)orc_sf_bytes(M, H, fmt, layout)); /* padding is zero */
    int err = 0;
#pragma omp parallel
    {
        float* h = (float*)malloc(sizeof(float) * H);
        float* y = (float*)malloc(sizeof(float) * H);
        uint8_t* codes = (uint8_t*)malloc((size_t)H);
        if (!h || !y || !codes) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < M; m++) {
                const uint16_t* xr = x + m * H;
                uint16_t* rr = residual + m * H;
                /* step 1 */
                for (int64_t i = 0; i < H; i++) {
                    volatile float s = wid(xr[i]) + wid(rr[i]);
                    h[i] = s;
                }
                /* step 2 */
                double S = 0.0;
                for (int64_t i = 0; i < H; i++) S += (double)h[i] * (double)h[i];
                double denom = sqrt(S / (double)H + (double)eps);
                float rstd = (float)(1.0 / denom);
                if (diag_rstd) diag_rstd[m] = rstd;
                /* residual write-back, then step 3 from the rounded copy */
                for (int64_t i = 0; i < H; i++) {
                    uint16_t hb = nar(h[i]);
                    rr[i] = hb;
                    volatile float t = wid(hb) * rstd;
                    volatile float yi = t * wid(w[i]);
                    y[i] = yi;
                }
                if (diag_y) memcpy(diag_y + m * H, y, sizeof(float) * H);
                /* step 4 */
                quant_row(y, m, H, fmt, gs, layout, out_packed + m * row_bytes(fmt, H), out_sf, codes,
                          diag_amax ? diag_amax + m * nblk : NULL,
                          diag_spre ? diag_spre + m * nblk : NULL,
                          diag_v ? diag_v + m * H : NULL);
            }
        }
        free(h); free(y); free(codes);
    }
    return err;
}

/* bf16 tensors (the page's default dtype). */
int orc_add_rmsnorm_quant(const uint16_t* x, uint16_t* residual, const uint16_t* w,
                          int64_t M, int64_t H, float eps, int fmt, int layout, float gs,
                          uint8_t* out_packed, uint8_t* out_sf,
                          float* diag_y, float* diag_v, float* diag_amax, float* diag_spre,
                          float* diag_rstd) {
    return orc_add_rmsnorm_quant_dt(x, residual, w, M, H, eps, fmt, layout, gs, out_packed, out_sf,
                                    diag_y, diag_v, diag_amax, diag_spre, diag_rstd, ORC_IN_BF16);
}

/* ------------------------------------------------------------------------- */
/* Quantize (FlashRT README: quantize_fp4_sfa_bf16)                            */
/* ------------------------------------------------------------------------- */
/* y_i = f32(x_i) (exact; x is bf16, or fp16 with dtype ORC_IN_F16 as in the
 * README's quantize_fp4_sfa_fp16), then the per-block rule above.  This makes
 * every GEMM operand: activations and the prepacked weights alike. */
int orc_quantize_dt(const uint16_t* x, int64_t rows, int64_t K, int fmt, int layout, float gs,
                    uint8_t* out_packed, uint8_t* out_sf, float* diag_spre, int dtype) {
    if (check_common(rows, K, fmt, layout)) return 1;
    if (dtype != ORC_IN_BF16 && dtype != ORC_IN_F16) return 1;
    const orc_widen_fn wid = widen_of(dtype);
    int64_t nblk = K / block_of(fmt);
    memset(out_sf, 0, (size_t)orc_sf_bytes(rows, K, fmt, layout));
    int err = 0;
#pragma omp parallel
    {
        float* y = (float*)malloc(sizeof(float) * K);
        uint8_t* codes = (uint8_t*)malloc((size_t)K);
        if (!y || !codes) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < rows; m++) {
                for (int64_t i = 0; i < K; i++) y[i] = wid(x[m * K + i]);
                quant_row(y, m, K, fmt, gs, layout, out_packed + m * row_bytes(fmt, K), out_sf, codes, NULL,
                          diag_spre ? diag_spre + m * nblk : NULL, NULL);
            }
        }
        free(y); free(codes);
    }
    return err;
}

int orc_quantize(const uint16_t* x, int64_t rows, int64_t K, int fmt, int layout, float gs,
                 uint8_t* out_packed, uint8_t* out_sf, float* diag_spre) {
    return orc_quantize_dt(x, rows, K, fmt, layout, gs, out_packed, out_sf, diag_spre, ORC_IN_BF16);
}

/* ------------------------------------------------------------------------- */
/* Dequantize (FlashRT README: dequantize_fp4_sfa_fp16)                       */
/* ------------------------------------------------------------------------- */
/* x_hat = fl32(E2M1(code) * scale / gs) for NVFP4 (gs divides: it was folded
 * into the block scale on the way in), E2M1(code) * 2^(b-127) for MXFP4,
 * E4M3(byte) * 2^(b-127) for MXFP8, then
 * stored as bf16, or as fp16 with dtype ORC_IN_F16 (the README's fp16
 * output), nearest-even either way (fp16: values from 65520 up become
 * infinity, small ones fp16 subnormals).  Also returns the binary64 values
 * when out_f64 is non-NULL. */
int orc_dequantize_dt(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K, int fmt,
                      int layout, float gs, uint16_t* out16, double* out_f64, int dtype) {
    if (check_common(rows, K, fmt, layout)) return 1;
    if (dtype != ORC_IN_BF16 && dtype != ORC_IN_F16) return 1;
    const orc_narrow_fn nar = narrow_of(dtype);
    int64_t B = block_of(fmt), nblk = K / B;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < rows; m++) {
        for (int64_t i = 0; i < K; i++) {
            uint8_t sb = sf[orc_sf_offset(m, i / B, nblk, fmt, layout)];
            double q;
            if (fmt == ORC_MXFP8) {
                q = orc_e4m3_value(packed[m * K + i]);
            } else {
                uint8_t byte = packed[m * (K / 2) + i / 2];
                q = orc_e2m1_value((i % 2 == 0) ? (byte & 15) : (byte >> 4));
            }
            /* q * scale is exact in binary64 (and in binary32) */
            double v = q * (e4m3_scaled(fmt) ? orc_e4m3_value(sb) : orc_ue8m0_value(sb));
            /* NVFP4: one division by gs; the binary64 quotient rounded to
             * binary32 equals the correctly rounded binary32 quotient */
            if (e4m3_scaled(fmt)) v = v / (double)gs;
            if (out_f64) out_f64[m * K + i] = v;
            if (out16) out16[m * K + i] = nar((float)v);
        }
    }
    return 0;
}

int orc_dequantize(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K, int fmt,
                   int layout, float gs, uint16_t* out_bf16, double* out_f64) {
    return orc_dequantize_dt(packed, sf, rows, K, fmt, layout, gs, out_bf16, out_f64, ORC_IN_BF16);
}

/* ------------------------------------------------------------------------- */
/* Inverse RoPE + MX quantization (vLLM page deepseek_v41/nvidia/ops/          */
/* fused_wo_a, FusedWoAKernel.device_kernel, the activation quant stage)       */
/* ------------------------------------------------------------------------- */
/*
 * x: bf16 (T, heads, D), one row of D elements per (token, head); the last R
 * elements of a row (from nope = D - R on) carry RoPE.  positions: (T) table
 * rows; rope: fp32 (P, R), each row cos[0 .. R/2) followed by sin[0 .. R/2).
 * For row (t, h), with pos = positions[t] (held to [0, P) -- the table is
 * never read outside) and each pair p of the rope slice, elements
 * k = nope + 2p and k + 1, c = rope[pos][p], s = rope[pos][p + R/2]:
 *     even' = even * c + odd * s          (the inverse rotation)
 *     odd'  = odd * c - even * s
 * each taken as the page's _rope_fma reads most plainly: the second product
 * rounded to fp32, then one fused multiply-add with the first.  Then each
 * 32-element block of the fp32 row is quantized with the page's floor on the
 * block maximum, amax' = max(amax, fl32(1e-10)), and the OCP MX rule on
 * amax' (the page's _scale is off-page; the same reading as the MX formats
 * elsewhere): e = clamp(floor(log2 amax') - emax, -127, 127), emax = 8 for
 * MXFP8 (E4M3 elements) and 2 for MXFP4 (E2M1), byte e + 127, elements
 * encode(y * 2^-e).  An all-zero block therefore gets e = -34 - emax, not the
 * zero byte of the other producers.  Diagnostics (optional): the rotated fp32
 * row values y (rows * D) and the floored block maxima (rows * D / 32).
 */
static float rope_term(float a, float c, float b, float s, int subtract) {
    volatile float bs = b * s;                   /* fl32(b * s) */
    return fmaf(a, c, subtract ? -bs : bs);      /* one rounding of a*c +- bs */
}

int orc_rope_quant(const uint16_t* x, const int64_t* positions, const float* rope, int64_t T,
                   int64_t heads, int64_t D, int64_t R, int64_t P, int fmt, int layout,
                   uint8_t* out_packed, uint8_t* out_sf, float* diag_y, float* diag_amax) {
    if (T < 0 || heads <= 0 || D <= 0 || D % 32 != 0 || R < 0 || R > D || R % 2 != 0) return 1;
    if (R > 0 && P <= 0) return 1;
    if (fmt != ORC_MXFP8 && fmt != ORC_MXFP4) return 1;
    if (check_common(T * heads, D, fmt, layout)) return 1;
    const int64_t rows = T * heads, nope = D - R, nblk = D / 32;
    const float floor_amax = 1e-10f;
    const int emax = (fmt == ORC_MXFP8) ? 8 : 2;
    memset(out_sf, 0, (size_t)orc_sf_bytes(rows, D, fmt, layout));
    int err = 0;
#pragma omp parallel
    {
        float* y = (float*)malloc(sizeof(float) * (size_t)D);
        uint8_t* codes = (uint8_t*)malloc((size_t)D);
        if (!y || !codes) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t row = 0; row < rows; row++) {
                const int64_t t = row / heads;
                for (int64_t k = 0; k < D; k++) y[k] = orc_bf16_to_f32(x[row * D + k]);
                if (R > 0) {
                    int64_t pos = positions[t];
                    if (pos < 0) pos = 0;
                    if (pos >= P) pos = P - 1;
                    for (int64_t p = 0; p < R / 2; p++) {
                        const int64_t k = nope + 2 * p;
                        const float c = rope[pos * R + p], s = rope[pos * R + p + R / 2];
                        const float even = y[k], odd = y[k + 1];
                        y[k] = rope_term(even, c, odd, s, 0);
                        y[k + 1] = rope_term(odd, c, even, s, 1);
                    }
                }
                if (diag_y) memcpy(diag_y + row * D, y, sizeof(float) * (size_t)D);
                for (int64_t b = 0; b < nblk; b++) {
                    float amax = 0.0f;
                    for (int i = 0; i < 32; i++) {
                        const float a = fabsf(y[b * 32 + i]);
                        if (a > amax) amax = a;
                    }
                    if (amax < floor_amax) amax = floor_amax;   /* the page's max(amax, 1e-10) */
                    if (diag_amax) diag_amax[row * nblk + b] = amax;
                    int E;
                    (void)frexp((double)amax, &E);              /* amax = f * 2^E, f in [0.5, 1) */
                    int e = (E - 1) - emax;                     /* floor(log2 amax) - emax */
                    if (e < -127) e = -127;
                    if (e > 127) e = 127;
                    out_sf[orc_sf_offset(row, b, nblk, fmt, layout)] = (uint8_t)(e + 127);
                    for (int i = 0; i < 32; i++) {
                        const float v = ldexpf(y[b * 32 + i], -e);
                        codes[b * 32 + i] = (fmt == ORC_MXFP8) ? orc_e4m3_encode(v) : orc_e2m1_encode(v);
                    }
                }
                pack_row(codes, D, fmt, out_packed + row * row_bytes(fmt, D));
            }
        }
        free(y);
        free(codes);
    }
    return err;
}

/* ------------------------------------------------------------------------- */
/* GEMM (FlashRT README: nvfp4_gemm_* family and its validation method)        */
/* ------------------------------------------------------------------------- */
/*
 * D[m,n] = alpha * sum_k Ahat[m,k] * Bhat[n,k], Ahat/Bhat dequantized exactly
 * (NVFP4, MXFP4, or MXFP8 with one E4M3 byte per element)
 * (no global scale: the caller folds 1/(gsA*gsB) into alpha), then
 *   bias:          + bias[n]
 *   residual:      + residual[m,n]
 *   bias+residual: + bias[n] + residual[m,n]
 *   bias+gelu:     GELU(z + bias[n]), GELU(t) = 0.5 t (1 + erf(t / sqrt 2))
 * all in binary64.  out_ref receives the unrounded value; out_l1 receives
 * |alpha| * sum_k |Ahat * Bhat| (the accumulation budget of the tolerance).
 */
static double dq(const uint8_t* packed, const uint8_t* sf, int64_t row, int64_t k, int64_t K,
                 int fmt, int layout) {
    int64_t B = block_of(fmt), nblk = K / B;
    uint8_t sb = sf[orc_sf_offset(row, k / B, nblk, fmt, layout)];
    double s = e4m3_scaled(fmt) ? orc_e4m3_value(sb) : orc_ue8m0_value(sb);
    if (fmt == ORC_MXFP8) return orc_e4m3_value(packed[row * K + k]) * s;   /* one byte per element */
    uint8_t byte = packed[row * (K / 2) + k / 2];
    uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
    return orc_e2m1_value(code) * s;
}

static double gelu_erf(double t) { return 0.5 * t * (1.0 + erf(t / sqrt(2.0))); }

static double epilogue(double acc, double alpha, int epi, const uint16_t* bias,
                       const uint16_t* residual, int64_t m, int64_t n, int64_t N) {
    double z = alpha * acc;
    if (epi == ORC_EPI_BIAS || epi == ORC_EPI_BIAS_RESIDUAL || epi == ORC_EPI_BIAS_GELU)
        z += (double)orc_bf16_to_f32(bias[n]);
    if (epi == ORC_EPI_RESIDUAL || epi == ORC_EPI_BIAS_RESIDUAL)
        z += (double)orc_bf16_to_f32(residual[m * N + n]);
    if (epi == ORC_EPI_BIAS_GELU) z = gelu_erf(z);
    return z;
}

/* Dequantize both operands once (fp64, exact), then a plain triple loop. */
int orc_gemm(const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
             int64_t M, int64_t N, int64_t K, int fmt, int layout_a, int layout_b, double alpha,
             int epi, const uint16_t* bias, const uint16_t* residual,
             double* out_ref, double* out_l1) {
    if (check_common(M, K, fmt, layout_a) || check_common(N, K, fmt, layout_b)) return 1;
    double* A = (double*)malloc(sizeof(double) * (size_t)(M * K));
    double* Bm = (double*)malloc(sizeof(double) * (size_t)(N * K));
    if (!A || !Bm) { free(A); free(Bm); return 2; }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++) A[m * K + k] = dq(a, sfa, m, k, K, fmt, layout_a);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) Bm[n * K + k] = dq(b, sfb, n, k, K, fmt, layout_b);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0, l1 = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = A[m * K + k] * Bm[n * K + k];
                acc += p;
                l1 += fabs(p);
            }
            out_ref[m * N + n] = epilogue(acc, alpha, epi, bias, residual, m, n, N);
            if (out_l1) out_l1[m * N + n] = fabs(alpha) * l1;
        }
    }
    free(A); free(Bm);
    return 0;
}

/* The same definition evaluated only at the listed (m, n) entries, for sampled
 * checks at sizes where the full product is too slow on the CPU. */
int orc_gemm_entries(const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                     int64_t M, int64_t N, int64_t K, int fmt, int layout_a, int layout_b,
                     double alpha, int epi, const uint16_t* bias, const uint16_t* residual,
                     int64_t count, const int64_t* idx_m, const int64_t* idx_n,
                     double* out_ref, double* out_l1) {
    if (check_common(M, K, fmt, layout_a) || check_common(N, K, fmt, layout_b)) return 1;
    for (int64_t t = 0; t < count; t++)
        if (idx_m[t] < 0 || idx_m[t] >= M || idx_n[t] < 0 || idx_n[t] >= N) return 1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; t++) {
        int64_t m = idx_m[t], n = idx_n[t];
        double acc = 0.0, l1 = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double p = dq(a, sfa, m, k, K, fmt, layout_a) * dq(b, sfb, n, k, K, fmt, layout_b);
            acc += p;
            l1 += fabs(p);
        }
        out_ref[t] = epilogue(acc, alpha, epi, bias, residual, m, n, N);
        if (out_l1) out_l1[t] = fabs(alpha) * l1;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* GEMM with bias + GELU epilogue emitting NVFP4 (FlashRT README:              */
/* nvfp4_gemm_bias_gelu_nvfp4 -- packed FP4 plus scales for the next GEMM)     */
/* ------------------------------------------------------------------------- */
/* t = alpha * acc + bias[n]; y = fl32(GELU(t)) (binary64 GELU rounded once);
 * then each 16-run of y along n is quantized with the NVFP4 block rule and
 * global scale gs_out, written as an (M, N) GEMM-A operand: packed (M, N/2)
 * and scales in out_layout.  Diagnostics (optional): y, v (M*N), l1 (M*N),
 * s_pre and amax (M*N/16). */
int orc_gemm_gelu_fp4(const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                      int64_t M, int64_t N, int64_t K, int fmt, int layout_a, int layout_b,
                      double alpha, const uint16_t* bias, float gs_out, int out_layout,
                      uint8_t* out_packed, uint8_t* out_sf,
                      float* diag_y, float* diag_v, double* diag_l1, float* diag_spre,
                      float* diag_amax) {
    if (check_common(M, K, fmt, layout_a) || check_common(N, K, fmt, layout_b)) return 1;
    /* NVFP4 or MXFP4 operands only: the output is NVFP4 for the next FP4 GEMM */
    if (fmt != ORC_NVFP4 && fmt != ORC_MXFP4) return 1;
    if (N % 16 != 0) return 1;
    double* ref = (double*)malloc(sizeof(double) * (size_t)(M * N));
    double* l1 = (double*)malloc(sizeof(double) * (size_t)(M * N));
    if (!ref || !l1) { free(ref); free(l1); return 2; }
    int rc = orc_gemm(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, ORC_EPI_BIAS_GELU,
                      bias, NULL, ref, l1);
    if (rc) { free(ref); free(l1); return rc; }
    int64_t nblk = N / 16;
    memset(out_sf, 0, (size_t)orc_sf_bytes(M, N, ORC_NVFP4, out_layout));
    int err = 0;
#pragma omp parallel
    {
        float* y = (float*)malloc(sizeof(float) * N);
        uint8_t* codes = (uint8_t*)malloc((size_t)N);
        if (!y || !codes) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < M; m++) {
                for (int64_t n = 0; n < N; n++) y[n] = (float)ref[m * N + n];
                if (diag_y) memcpy(diag_y + m * N, y, sizeof(float) * N);
                quant_row(y, m, N, ORC_NVFP4, gs_out, out_layout, out_packed + m * (N / 2), out_sf,
                          codes, diag_amax ? diag_amax + m * nblk : NULL,
                          diag_spre ? diag_spre + m * nblk : NULL, diag_v ? diag_v + m * N : NULL);
            }
        }
        free(y); free(codes);
    }
    if (diag_l1) memcpy(diag_l1, l1, sizeof(double) * (size_t)(M * N));
    free(ref); free(l1);
    return err;
}

/* ------------------------------------------------------------------------- */
/* GEMM with FP8 output quantization (vLLM page deepseek_v41/nvidia/ops/       */
/* fused_wo_a, FusedWoAKernel.device_kernel, its output epilogue)             */
/* ------------------------------------------------------------------------- */
/* Round a binary64 to bf16 (8 significant bits, binary32's exponent range),
 * nearest-even, in one step from the exact value: count the value in steps
 * of its binade's bf16 grid (2^(E-7), 2^-133 below 2^-126) and round the
 * count.  Returns the bf16 value as a binary32 (exact). */
static float f64_to_bf16_value(double v) {
    double a = fabs(v);
    if (a == 0.0) return (float)v;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                          /* floor(log2 a) */
    if (E < -126) E = -126;                  /* subnormal grid: 2^-133 */
    double q = rint(ldexp(a, 7 - E));        /* count of 2^(E-7) steps, ties to even */
    double r = ldexp(q, E - 7);
    return (float)(v < 0 ? -r : r);
}

/* value[m,n] = bf16(alpha * acc[m,n]) -- the page rounds the reduced sum to
 * bf16 before quantizing -- then each 32-run of a row along n is quantized as
 * MXFP8 (the MX rule of quant_block: OCP scale with emax 8, an all-zero block
 * gets byte 0; E4M3 elements nearest-even, saturating, sign kept), one byte
 * an element into out_packed (M, N) and the scale bytes in out_layout:
 * LINEAR, or the page's 128 x 4 swizzle (its F8_128x4 scale bytes).
 * Diagnostics (optional): the unrounded binary64 values and their L1 budget. */
int orc_gemm_fp8_out(const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                     int64_t M, int64_t N, int64_t K, int fmt, int layout_a, int layout_b,
                     double alpha, int out_layout, uint8_t* out_packed, uint8_t* out_sf,
                     double* diag_ref, double* diag_l1) {
    if (check_common(M, K, fmt, layout_a) || check_common(N, K, fmt, layout_b)) return 1;
    if (N % 32 != 0) return 1;
    if (out_layout != ORC_SF_LINEAR && out_layout != ORC_SF_SWZ128) return 1;
    double* ref = (double*)malloc(sizeof(double) * (size_t)(M * N));
    double* l1 = (double*)malloc(sizeof(double) * (size_t)(M * N));
    if (!ref || !l1) { free(ref); free(l1); return 2; }
    int rc = orc_gemm(a, b, sfa, sfb, M, N, K, fmt, layout_a, layout_b, alpha, ORC_EPI_NONE, NULL, NULL,
                      ref, l1);
    if (rc) { free(ref); free(l1); return rc; }
    memset(out_sf, 0, (size_t)orc_sf_bytes(M, N, ORC_MXFP8, out_layout));
    int err = 0;
#pragma omp parallel
    {
        float* y = (float*)malloc(sizeof(float) * (size_t)N);
        uint8_t* codes = (uint8_t*)malloc((size_t)N);
        if (!y || !codes) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < M; m++) {
                for (int64_t n = 0; n < N; n++) y[n] = f64_to_bf16_value(ref[m * N + n]);
                quant_row(y, m, N, ORC_MXFP8, 1.0f, out_layout, out_packed + m * N, out_sf, codes, NULL, NULL,
                          NULL);
            }
        }
        free(y);
        free(codes);
    }
    if (diag_ref) memcpy(diag_ref, ref, sizeof(double) * (size_t)(M * N));
    if (diag_l1) memcpy(diag_l1, l1, sizeof(double) * (size_t)(M * N));
    free(ref);
    free(l1);
    return err;
}

/* E4M3 codes of MX blocks of 32 values under given scale bytes (the parity
 * checker's re-encoding of candidate values, one call for many blocks). */
void orc_mxfp8_encode_blocks(const float* y, int64_t nblocks, const uint8_t* sbytes, uint8_t* codes) {
    for (int64_t b = 0; b < nblocks; b++)
        orc_encode_with_scale(y + b * 32, 32, ORC_MXFP8, 1.0f, sbytes[b], codes + b * 32, NULL);
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the following calls use (the timing of the oracle on one core and
 * on all of them); n < 1 is ignored. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
