#pragma once
// gemm_kernels.hpp -- block-scaled A4W4 GEMM for gfx950,
// out = epilogue(alpha * A . B^T): the kernels and their launch templates,
// instantiated per (format, epilogue) in the gemm_inst_*.hip units and
// dispatched by gemm.hip (FlashRT fp4-gemm README: nvfp4_gemm_bf16 and its epilogue family, the
// "Tensor Contract": A (M, K/2) and B (N, K/2) packed FP4 plus block scales).
//
// Contraction unit.  K is walked in "supersteps" of 256 elements (128 packed
// bytes per row), each made of two 128-element stages h = 0, 1.  Lane (r, c)
// of a wave (r = lane % 32, c = lane / 32) owns, of row r, bytes
// 64h + 32c .. 64h + 32c + 31 of every superstep; its quarter Q = 2h + s is
// the 16 bytes at 64h + 32c + 16s.  A sum over K may be taken in any order as
// long as A and B agree, so both operands use this same assignment:
//   MXFP4: four v_mfma_scale_f32_32x32x64_f8f6f4 per superstep; quarter Q
//          feeds the lane's 32-element block 4h + 2c + s of the superstep,
//          whose UE8M0 scale is byte Q of the lane's scale word (selected by
//          the instruction's op_sel).  One 32-bit word per lane therefore
//          feeds the four MFMAs -- the TILED scale layout stores exactly
//          these words, 32 rows x 2 lane halves per 256-byte group.
//   NVFP4: E4M3 16-block scales have no native MFMA form, so each FP4 value
//          is multiplied by its block scale in fp16 -- exact, since E2M1 times
//          E4M3 has at most 6 significant bits and lies in [2^-10, 2688] --
//          and sixteen v_mfma_f32_32x32x16_f16 consume the superstep; dword t'
//          of quarter Q is one step, block 8h + 4c + 2s + t'/2.
// Accumulation is fp32 in the MFMA accumulators.
//
// Schedules:
//   prefill: 256x256 macro tiles, 4 waves of 128x128; A and B supersteps are
//            copied to LDS by buffer loads that write LDS directly (two
//            buffers, 16-byte chunks XOR-swizzled by row so the 32-row
//            fragment reads are bank-conflict free); tiles are mapped so that
//            consecutive tiles share an XCD's L2.
//            NVFP4 (K % 64 == 0) and MXFP8 (K % 128 == 0) run the 128 x 384
//            schedule of gemm_nv.hpp instead, which converts each activation
//            fragment once per workgroup.
//   decode:  the weights are the MFMA row operand (32 weight rows per
//            workgroup, all <= 128 tokens as the column operand, so each weight
//            byte is read once); the K supersteps are dealt round-robin to the
//            workgroup's waves and the partial tiles summed through LDS.
//   split-K: the decode schedule (<= 128 tokens) or the 128 x 384 one
//            (NVFP4 above 64 tokens; NVFP4 / MXFP8 prefill shapes with few
//            tiles) with K split across workgroups, fp32 partials in a
//            workspace, summed in a fixed order by gemm_splitk_reduce_kernel,
//            which applies the epilogue.
// Epilogues run per 32x32 tile through LDS so that every global access is a
// contiguous 16-element run of a row: bf16 out with alpha, bias, residual,
// GELU; or GELU followed by NVFP4 quantization along N (FP4 output for the
// next GEMM).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace lowbit {
namespace gk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSSBytes = 128;   // packed bytes per row per superstep (256 FP4 / 128 FP8 elements)
// elements of K in one superstep, and packed bytes per K element times 2
template <int FMT> constexpr int ss_elems() { return FMT == kMXFP8 ? 128 : 256; }
template <int FMT> constexpr int64_t row_bytes(int64_t K) { return FMT == kMXFP8 ? K : K / 2; }
constexpr int kEpiPitch = 36;   // fp32 pitch of a 32x32 epilogue tile in LDS

// 64 bytes of one row held by one lane for one superstep.
struct Frag {
  u32x4 q[4];
};

// A lane's scale bytes for one superstep: MXFP4 4 bytes (blocks 2c, 2c+1,
// 2c+4, 2c+5 of the superstep's 8, byte Q for quarter Q); NVFP4 8 bytes
// (blocks 4c..4c+3 then 8+4c..8+4c+3 of its 16, byte 2Q + t'/2).  In the
// TILED layout each of these words is one aligned word of the scale buffer.
template <int FMT> struct SfWord;
template <> struct SfWord<kMXFP4> { uint32_t w; };
template <> struct SfWord<kNVFP4> { uint32_t w[2]; };
// MXFP8: a 128-element superstep holds four 32-blocks; lane half c takes
// blocks c (bytes 0..31 of its 64) and 2 + c (bytes 64..95): byte h of the
// word is the UE8M0 scale of block 2h + c (LINEAR scales only)
template <> struct SfWord<kMXFP8> { uint32_t w; };

// byte-select pattern of v_perm picking bytes {2c, 2c+1} of two words
__device__ __forceinline__ uint32_t pair_sel(int c) { return c ? 0x07060302u : 0x05040100u; }

template <int FMT>
__device__ __forceinline__ void load_sf_fp4(SfWord<FMT>& out, const uint8_t* sf, int layout, int64_t row,
                                        int64_t R, int64_t nblk, int64_t ss, int c) {
  // absent rows / blocks carry no data; give them a harmless finite scale
  constexpr uint32_t kPad = (FMT == kMXFP4) ? 0x7F7F7F7Fu : 0u;
  constexpr int NW = (FMT == kMXFP4) ? 1 : 2;
  uint32_t w[NW];
#pragma unroll
  for (int i = 0; i < NW; i++) w[i] = kPad;
  if (row < R) {
    const int64_t ktiles = (nblk + 7) >> 3;
    if (layout == kTiled) {
      if constexpr (FMT == kMXFP4) {
        w[0] = *reinterpret_cast<const uint32_t*>(sf + (((row >> 5) * ktiles + ss) << 8) +
                                                  ((c * 32 + (row & 31)) << 2));
      } else {
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int64_t tile = 2 * ss + h;
          if (tile < ktiles)
            w[h] = *reinterpret_cast<const uint32_t*>(sf + (((row >> 5) * ktiles + tile) << 8) +
                                                      ((c * 32 + (row & 31)) << 2));
        }
      }
    } else {
      const uint8_t* p = sf + row * nblk;
#pragma unroll
      for (int j = 0; j < 4 * NW; j++) {
        // MXFP4 byte j <-> block 8ss + 2c + (j&1) + 4(j>>1); NVFP4 byte j <-> 16ss + 8(j/4) + 4c + j%4
        const int64_t kb = (FMT == kMXFP4) ? 8 * ss + 2 * c + (j & 1) + 4 * (j >> 1)
                                           : 16 * ss + 8 * (j >> 2) + 4 * c + (j & 3);
        const uint32_t byte = (kb < nblk) ? (uint32_t)p[kb] : (kPad & 0xFF);
        w[j >> 2] = (w[j >> 2] & ~(0xFFu << (8 * (j & 3)))) | (byte << (8 * (j & 3)));
      }
    }
  }
  if constexpr (FMT == kMXFP4) {
    out.w = w[0];
  } else {
    out.w[0] = w[0];
    out.w[1] = w[1];
  }
}

// MXFP8 (LINEAR scales): byte h of the lane's word is the scale of block
// 2h + c of superstep ss; absent rows / blocks get 2^0
__device__ __forceinline__ void load_sf_f8(SfWord<kMXFP8>& out, const uint8_t* sf, int64_t row, int64_t R,
                                           int64_t nblk, int64_t ss, int c) {
  uint32_t w = 0x7F7Fu;
  if (row < R) {
    const uint8_t* p = sf + row * nblk;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int64_t kb = 4 * ss + 2 * h + c;
      const uint32_t byte = (kb < nblk) ? (uint32_t)p[kb] : 0x7Fu;
      w = (w & ~(0xFFu << (8 * h))) | (byte << (8 * h));
    }
  }
  out.w = w;
}

template <int FMT>
__device__ __forceinline__ void load_sf(SfWord<FMT>& out, const uint8_t* sf, int layout, int64_t row,
                                        int64_t R, int64_t nblk, int64_t ss, int c) {
  if constexpr (FMT == kMXFP8) {
    (void)layout;
    load_sf_f8(out, sf, row, R, nblk, ss, c);
    return;
  } else {
    load_sf_fp4<FMT>(out, sf, layout, row, R, nblk, ss, c);
  }
}

// byte offset of quarter Q of lane half c inside a superstep's 128 bytes
__device__ __forceinline__ int quarter_off(int Q, int c) { return 64 * (Q >> 1) + 32 * c + 16 * (Q & 1); }

// the 64 packed bytes lane half c owns of `row` in superstep ss; zero outside.
// Plain cached loads for both operands: a lane's four 16-byte loads share
// 128-byte lines with the other lane half, and nontemporal loads of the
// weights were measured 15-30% slower on every decode shape (same HBM bytes).
// NVFP4 rows with K % 32 == 16 are 8 mod 16 bytes long: their rows start on
// 8-byte boundaries and their last 16-element block fills only the first
// half of a 16-byte chunk, so those rows are read in naturally aligned 8-byte
// halves, the half past the row end reading as zero (HALF: K/2 % 16 == 8).
template <bool HALF = false>
__device__ __forceinline__ void load_frag_global(Frag& f, const uint8_t* base, int64_t row, int64_t R,
                                                 int64_t kbytes, int64_t ss, int c) {
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const int64_t o = ss * kSSBytes + quarter_off(s, c);
    const uint8_t* p = base + row * kbytes + o;
    if constexpr (HALF) {
      const uint2 z2 = {0u, 0u};
      const uint2 lo = (row < R && o + 8 <= kbytes) ? *reinterpret_cast<const uint2*>(p) : z2;
      const uint2 hi = (row < R && o + 16 <= kbytes) ? *reinterpret_cast<const uint2*>(p + 8) : z2;
      f.q[s] = u32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      if (row < R && o + 16 <= kbytes)
        f.q[s] = *reinterpret_cast<const u32x4*>(p);
      else
        f.q[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ v8i as_v8i(u32x4 q) {
  return v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
}

// Scaled FP4 MFMA, slice S of a superstep (op_sel must be a constant).
template <int S>
__device__ __forceinline__ v16f mfma_mx(u32x4 a, u32x4 b, v16f acc, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_v8i(a), as_v8i(b), acc, 4, 4, S, (int)sa, S,
                                                         (int)sb);
}

// Scaled FP8 (E4M3) MFMA: a lane's 32 bytes are the two 16-byte halves a0, a1
// (b0, b1); scale byte S of sa / sb.  SWAP: B is the row operand, so the
// accumulator holds the transposed tile (the split-K partial layout).
template <int S, bool SWAP>
__device__ __forceinline__ v16f mfma_f8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, v16f acc, uint32_t sa,
                                        uint32_t sb) {
  const v8i a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const v8i b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  if constexpr (SWAP) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc, 0, 0, S, (int)sb, S, (int)sa);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, S, (int)sa, S, (int)sb);
}

// NVFP4 dequantization to fp16, exact.  An E2M1 value (2 significant bits)
// times an E4M3 scale (4 significant bits) has at most 6 significant bits and
// lies in [2^-10, 2688], so it is an fp16 normal number.  The E4M3 byte is
// decoded by the FP8 conversion and split into its power of two p (what the
// scaled FP4->fp16 conversion applies: that conversion uses only the exponent
// of its fp32 scale) and its sign-carrying mantissa m = +-1.mmm (applied by
// one packed fp16 multiply, exact).  A zero scale gives p = 0 and zeros.
struct NvPart {
  float p;   // 2^e of the block scale (0 for a zero scale)
  v2h m;     // sign * 1.mmm, in both halves
};
__device__ __forceinline__ NvPart nv_part(const SfWord<kNVFP4>& sw, int blk) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)(sw.w[blk >> 2] >> (8 * (blk & 3))), 0);
  const uint32_t u = __float_as_uint(s);
  const _Float16 h = (_Float16)__uint_as_float((u & 0x807FFFFFu) | 0x3F800000u);
  return NvPart{__uint_as_float(u & 0x7F800000u), v2h{h, h}};
}
// Eight E2M1 codes (one dword, element i in nibble i) times the block scale.
__device__ __forceinline__ v8h dq8(uint32_t w, NvPart sc) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p, 0) * sc.m;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p, 1) * sc.m;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p, 2) * sc.m;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p, 3) * sc.m;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// MXFP8 dequantization to bf16, exact while the product is a normal bf16:
// an E4M3 value has 4 significant bits and the UE8M0 scale is a power of two
// 2^e, so E4M3 * 2^e is exact for e in [-117, 119] (bf16 has binary32's
// exponent range).  Eight elements (two dwords, element i in byte i).
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v8bf dq8_f8(uint32_t lo, uint32_t hi, float scale) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, scale, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, scale, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, scale, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, scale, true);
  return v8bf{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
// UE8M0 scale byte h of an MXFP8 scale word as an fp32 power of two
__device__ __forceinline__ float f8_scale(const SfWord<kMXFP8>& sw, int h) {
  return ue8m0_to_f32((sw.w >> (8 * h)) & 0xFFu);
}
// acc[i][j] += quarter S of an MXFP8 superstep: 16 elements of block 2(S/2) + c
// per lane, two bf16 MFMA steps of 8
template <int S, int TI, int TJ>
__device__ __forceinline__ void quarter_f8(v16f (&acc)[TI][TJ], const u32x4 (&qa)[TI], const u32x4 (&qb)[TJ],
                                           const SfWord<kMXFP8> (&sa)[TI], const SfWord<kMXFP8> (&sb)[TJ]) {
  float fa[TI], fb[TJ];
#pragma unroll
  for (int i = 0; i < TI; i++) fa[i] = f8_scale(sa[i], S >> 1);
#pragma unroll
  for (int j = 0; j < TJ; j++) fb[j] = f8_scale(sb[j], S >> 1);
#pragma unroll
  for (int t = 0; t < 2; t++) {
    v8bf va[TI], vb[TJ];
#pragma unroll
    for (int i = 0; i < TI; i++) va[i] = dq8_f8(qa[i][2 * t], qa[i][2 * t + 1], fa[i]);
#pragma unroll
    for (int j = 0; j < TJ; j++) vb[j] = dq8_f8(qb[j][2 * t], qb[j][2 * t + 1], fb[j]);
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
      for (int j = 0; j < TJ; j++)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], vb[j], acc[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t frag_dword(const Frag& f, int t) {
  const u32x4 q = f.q[t >> 2];
  switch (t & 3) {
    case 0: return q.x;
    case 1: return q.y;
    case 2: return q.z;
    default: return q.w;
  }
}

// acc[i][j] += A-frag i x B-frag j over one superstep.
template <int FMT, int TI, int TJ>
__device__ __forceinline__ void superstep_mma(v16f (&acc)[TI][TJ], const Frag (&fa)[TI], const Frag (&fb)[TJ],
                                              const SfWord<FMT> (&sa)[TI], const SfWord<FMT> (&sb)[TJ]) {
  if constexpr (FMT == kMXFP8) {
    u32x4 qa[TI], qb[TJ];
#define LB_F8(S)                                                                                     \
    _Pragma("unroll") for (int i = 0; i < TI; i++) qa[i] = fa[i].q[S];                              \
    _Pragma("unroll") for (int j = 0; j < TJ; j++) qb[j] = fb[j].q[S];                              \
    quarter_f8<S, TI, TJ>(acc, qa, qb, sa, sb);
    LB_F8(0) LB_F8(1) LB_F8(2) LB_F8(3)
#undef LB_F8
  } else if constexpr (FMT == kMXFP4) {
#define LB_SLICE(S)                                                                                  \
    _Pragma("unroll") for (int i = 0; i < TI; i++)                                                   \
    _Pragma("unroll") for (int j = 0; j < TJ; j++)                                                   \
      acc[i][j] = mfma_mx<S>(fa[i].q[S], fb[j].q[S], acc[i][j], sa[i].w, sb[j].w);
    LB_SLICE(0) LB_SLICE(1) LB_SLICE(2) LB_SLICE(3)
#undef LB_SLICE
  } else {
#pragma unroll
    for (int t = 0; t < 16; t++) {
      v8h va[TI], vb[TJ];
#pragma unroll
      for (int i = 0; i < TI; i++) va[i] = dq8(frag_dword(fa[i], t), nv_part(sa[i], t >> 1));
#pragma unroll
      for (int j = 0; j < TJ; j++) vb[j] = dq8(frag_dword(fb[j], t), nv_part(sb[j], t >> 1));
#pragma unroll
      for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i], vb[j], acc[i][j], 0, 0, 0);
    }
  }
}

// MXFP8 on the 128-byte-stage prefill schedule: step Q of a superstep (128
// FP8 elements of a row, 32-element blocks 4s .. 4s + 3 of superstep s) is one
// scaled FP8 MFMA per tile pair.  The instruction's first K block is the
// first 16 bytes (x0) of both lane halves, its second the last 16 (x1), and
// lane half c supplies the scale of block c: so x0 of lane half c is the
// 16 bytes [16c, 16c + 16) of block 2Q and x1 those of block 2Q + 1 (the
// fragments of the stage's quarters 2Q and 2Q + 1), and lane half c's scale
// word, shifted by 8c, holds block 2Q + c at byte 2Q.
// (SW: the scale word type; only SfWord<kMXFP8> reaches a launch)
template <int Q, bool SWAP, int TI, int TJ, class SW>
__device__ __forceinline__ void step_f8(v16f (&acc)[TI][TJ], const u32x4 (&a0)[TI], const u32x4 (&a1)[TI],
                                        const u32x4 (&b0)[TJ], const u32x4 (&b1)[TJ], const SW (&sa)[TI],
                                        const SW (&sb)[TJ]) {
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++)
      acc[i][j] = mfma_f8<2 * Q, SWAP>(a0[i], a1[i], b0[j], b1[j], acc[i][j], sa[i].w, sb[j].w);
}

// Exact MXFP8 on the 128-byte-stage prefill schedule: quarter S of a superstep
// holds, in both lane halves, 16 bytes of its 32-element block S (bytes
// [16c, 16c + 16)), widened exactly to bf16 with that block's power of two
// (byte S of the unshifted scale word), two bf16 MFMA steps of 8 elements a
// lane.  SWAP: B as the row operand (split-K partials).
template <int S, bool SWAP, int TI, int TJ, class SW>
__device__ __forceinline__ void quarter_f8dq(v16f (&acc)[TI][TJ], const u32x4 (&qa)[TI], const u32x4 (&qb)[TJ],
                                             const SW (&sa)[TI], const SW (&sb)[TJ]) {
  float fa[TI], fb[TJ];
#pragma unroll
  for (int i = 0; i < TI; i++) fa[i] = ue8m0_to_f32((sa[i].w >> (8 * S)) & 0xFFu);
#pragma unroll
  for (int j = 0; j < TJ; j++) fb[j] = ue8m0_to_f32((sb[j].w >> (8 * S)) & 0xFFu);
#pragma unroll
  for (int t = 0; t < 2; t++) {
    v8bf va[TI], vb[TJ];
#pragma unroll
    for (int i = 0; i < TI; i++) va[i] = dq8_f8(qa[i][2 * t], qa[i][2 * t + 1], fa[i]);
#pragma unroll
    for (int j = 0; j < TJ; j++) vb[j] = dq8_f8(qb[j][2 * t], qb[j][2 * t + 1], fb[j]);
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
      for (int j = 0; j < TJ; j++)
        acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[j], va[i], acc[i][j], 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], vb[j], acc[i][j], 0, 0, 0);
  }
}

// acc[i][j] += quarter S (bytes 16S..16S+15 of each lane's 64) of a superstep:
// MXFP4 one scaled MFMA per tile pair (op_sel S picks the block's scale
// byte); NVFP4 four fp16 MFMA steps (block 8c + 2S + t/2).
template <int FMT, int S, int TI, int TJ>
__device__ __forceinline__ void quarter_mma(v16f (&acc)[TI][TJ], const u32x4 (&qa)[TI], const u32x4 (&qb)[TJ],
                                            const SfWord<FMT> (&sa)[TI], const SfWord<FMT> (&sb)[TJ]) {
  if constexpr (FMT == kMXFP8) {
    quarter_f8<S, TI, TJ>(acc, qa, qb, sa, sb);
  } else if constexpr (FMT == kMXFP4) {
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
      for (int j = 0; j < TJ; j++) acc[i][j] = mfma_mx<S>(qa[i], qb[j], acc[i][j], sa[i].w, sb[j].w);
  } else {
#pragma unroll
    for (int t = 0; t < 4; t++) {
      v8h va[TI], vb[TJ];
#pragma unroll
      for (int i = 0; i < TI; i++) va[i] = dq8(qa[i][t], nv_part(sa[i], 2 * S + (t >> 1)));
#pragma unroll
      for (int j = 0; j < TJ; j++) vb[j] = dq8(qb[j][t], nv_part(sb[j], 2 * S + (t >> 1)));
#pragma unroll
      for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i], vb[j], acc[i][j], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// FP4-out epilogue of one 16-element NVFP4 block of output row m (columns
// n .. n+15, n a multiple of 16): GELU of the pre-activations z, the block
// scale with the output global scale gs, codes and scale byte stored.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gelu_fp4_block(const float (&z)[16], int64_t m, int64_t n, const GemmArgs& g,
                                               float gs) {
  float y[16];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    y[k] = gelu_erf(z[k]);
    amax = fmaxf(amax, fabsf(y[k]));
  }
  float inv;
  const uint32_t sb = nv_block_scale(amax, gs, &inv);
#pragma unroll
  for (int k = 0; k < 16; k++) y[k] = __fmul_rn(y[k], inv);
  uint2 p;
  p.x = e2m1x8(y);
  p.y = e2m1x8(y + 8);
  *reinterpret_cast<uint2*>(g.out_packed + m * (g.N / 2) + n / 2) = p;
  g.out_sf[sf_offset(kNVFP4, g.out_layout, m, n / 16, g.N / 16)] = (uint8_t)sb;
}

// ---------------------------------------------------------------------------
// Epilogue on one 16-element run of output row m (columns n .. n+15), values
// from LDS.  n is a multiple of 16.
// ---------------------------------------------------------------------------
template <int EPI>
__device__ __forceinline__ void epi_run16(const float* t, int64_t m, int64_t n, const GemmArgs& g) {
  if (m >= g.M || n >= g.N) return;
  const float alpha = g.alpha;
  if constexpr (EPI == kEpiFp8) {
    // FP8 output ([WOA] FusedWoAKernel epilogue): bf16(alpha * acc) first, then
    // the 32-column MX block: this lane's 16 columns and its partner's (lane
    // ^ 32, the same row and the other half of the block: every caller maps
    // the two halves of a 32-column tile onto lanes l and l + 32, and N % 32
    // == 0 keeps both halves live together) share one OCP MX scale (emax 8)
    float y[16];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; k++) {
      y[k] = bf16_to_f32(f32_to_bf16(alpha * t[k]));
      amax = fmaxf(amax, fabsf(y[k]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
    float inv;
    const uint32_t sb = mx_block_scale_e<8>(amax, &inv);
#pragma unroll
    for (int k = 0; k < 16; k++) y[k] = __fmul_rn(y[k], inv);   // exact: a power of two
    const uint2 lo = e4m3x8(y), hi = e4m3x8(y + 8);
    *reinterpret_cast<uint4*>(g.out_packed + m * g.N + n) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    if ((n & 31) == 0) g.out_sf[sf_offset(kMXFP8, g.out_layout, m, n / 32, g.N / 32)] = (uint8_t)sb;
  } else if constexpr (EPI == kEpiBiasGeluFp4) {
    // N % 16 == 0, so the whole block is in range
    float z[16];
#pragma unroll
    for (int k = 0; k < 16; k++) z[k] = alpha * t[k] + bf16_to_f32(g.bias[n + k]);
    gelu_fp4_block(z, m, n, g, g.gs_out ? *g.gs_out : 1.0f);
  } else {
    const bool vec = (g.N % 8) == 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int64_t nn = n + 8 * h;
      if (nn >= g.N) break;
      float z[8];
#pragma unroll
      for (int k = 0; k < 8; k++) z[k] = alpha * t[8 * h + k];
      if (vec && nn + 8 <= g.N) {
        if constexpr (EPI == kEpiBias || EPI == kEpiBiasResidual || EPI == kEpiBiasGelu) {
          const uint4 bv = *reinterpret_cast<const uint4*>(g.bias + nn);
          const uint32_t* bw = reinterpret_cast<const uint32_t*>(&bv);
#pragma unroll
          for (int k = 0; k < 4; k++) { z[2 * k] += bf16_lo(bw[k]); z[2 * k + 1] += bf16_hi(bw[k]); }
        }
        if constexpr (EPI == kEpiResidual || EPI == kEpiBiasResidual) {
          const uint4 rv = *reinterpret_cast<const uint4*>(g.residual + m * g.N + nn);
          const uint32_t* rw = reinterpret_cast<const uint32_t*>(&rv);
#pragma unroll
          for (int k = 0; k < 4; k++) { z[2 * k] += bf16_lo(rw[k]); z[2 * k + 1] += bf16_hi(rw[k]); }
        }
        if constexpr (EPI == kEpiBiasGelu) {
#pragma unroll
          for (int k = 0; k < 8; k++) z[k] = gelu_erf(z[k]);
        }
        uint4 o;
        o.x = pack_bf16x2(z[0], z[1]);
        o.y = pack_bf16x2(z[2], z[3]);
        o.z = pack_bf16x2(z[4], z[5]);
        o.w = pack_bf16x2(z[6], z[7]);
        *reinterpret_cast<uint4*>(g.out + m * g.N + nn) = o;
      } else {
#pragma unroll
        for (int k = 0; k < 8; k++) {
          if (nn + k >= g.N) continue;   // unrolled with a predicate: z stays in registers
          float v = z[k];
          if constexpr (EPI == kEpiBias || EPI == kEpiBiasResidual || EPI == kEpiBiasGelu)
            v += bf16_to_f32(g.bias[nn + k]);
          if constexpr (EPI == kEpiResidual || EPI == kEpiBiasResidual)
            v += bf16_to_f32(g.residual[m * g.N + nn + k]);
          if constexpr (EPI == kEpiBiasGelu) v = gelu_erf(v);
          g.out[m * g.N + nn + k] = f32_to_bf16(v);
        }
      }
    }
  }
}

// Zero the padding of the FP8 output's 128 x 4 scale layout that this
// workgroup owns: rows [max(M, r0), min(rows_pad, r1)) x blocks [b0, b1), and,
// for the workgroup holding the last column block, blocks [nblk, nblk_pad)
// of rows [r0, min(rows_pad, r1)).
__device__ __forceinline__ void fp8_out_padding(const GemmArgs& g, int64_t r0, int64_t r1, int64_t b0,
                                                int64_t b1, bool last_col_tile, int tid, int nthreads) {
  if (g.out_layout != kSwz128) return;
  const int64_t nblk = g.N / 32;
  const int64_t nblk_pad = sf_pad_blocks(kSwz128, nblk);
  const int64_t rows_pad = sf_pad_rows(kSwz128, g.M);
  const int64_t re = r1 < rows_pad ? r1 : rows_pad;
  const int64_t be = b1 < nblk ? b1 : nblk;
  const int64_t rs = r0 > g.M ? r0 : g.M;
  if (rs < re && b0 < be) {
    const int64_t cnt = (re - rs) * (be - b0);
    for (int64_t i = tid; i < cnt; i += nthreads)
      g.out_sf[sf_offset(kMXFP8, kSwz128, rs + i / (be - b0), b0 + i % (be - b0), nblk)] = 0;
  }
  if (last_col_tile && nblk_pad > nblk && r0 < re) {
    const int64_t w = nblk_pad - nblk;
    const int64_t cnt = (re - r0) * w;
    for (int64_t i = tid; i < cnt; i += nthreads)
      g.out_sf[sf_offset(kMXFP8, kSwz128, r0 + i / w, nblk + i % w, nblk)] = 0;
  }
}

// Zero the TILED padding of the FP4 output scales that this workgroup owns:
// rows [max(M, r0), min(rows_pad, r1)) x blocks [b0, b1), and, for the
// workgroup holding the last column block, blocks [nblk, nblk_pad) of rows
// [r0, min(rows_pad, r1)).
__device__ __forceinline__ void fp4_out_padding(const GemmArgs& g, int64_t r0, int64_t r1, int64_t b0,
                                                int64_t b1, bool last_col_tile, int tid, int nthreads) {
  if (g.out_layout != kTiled) return;
  const int64_t nblk = g.N / 16;
  const int64_t nblk_pad = (nblk + 7) / 8 * 8;
  const int64_t rows_pad = (g.M + 31) / 32 * 32;
  const int64_t re = r1 < rows_pad ? r1 : rows_pad;
  const int64_t be = b1 < nblk ? b1 : nblk;
  const int64_t rs = r0 > g.M ? r0 : g.M;
  if (rs < re && b0 < be) {
    const int64_t cnt = (re - rs) * (be - b0);
    for (int64_t i = tid; i < cnt; i += nthreads)
      g.out_sf[sf_offset(kNVFP4, kTiled, rs + i / (be - b0), b0 + i % (be - b0), nblk)] = 0;
  }
  if (last_col_tile && nblk_pad > nblk && r0 < re) {
    const int64_t w = nblk_pad - nblk;
    const int64_t cnt = (re - r0) * w;
    for (int64_t i = tid; i < cnt; i += nthreads)
      g.out_sf[sf_offset(kNVFP4, kTiled, r0 + i / w, nblk + i % w, nblk)] = 0;
  }
}

// Epilogue of one wave's TI x TJ grid of 32x32 accumulator tiles, staged
// through the wave's LDS area (32 rows x kEpiRowPitch floats).
//  * bf16 outputs with N % 8 == 0: a whole row block (32 rows x 32*TJ
//    columns) is written to LDS, then lane l takes 8 consecutive columns
//    (l % 16) * 8 of rows 4q + l / 16, q = 0..7, so every residual load and
//    every output store instruction covers four full 2*32*TJ-byte row
//    segments.  The bias is loaded once (it depends on the column only); the
//    next row block's residual is loaded while this one is combined.  The
//    pitch 32*TJ + 8 puts the two lane halves of an accumulator write on
//    disjoint banks.
//  * FP4 out: the same row-block staging; a lane takes 16-column NVFP4
//    blocks of one row.
//  * otherwise (ragged N) tile by tile through epi_run16, a lane holding 16
//    consecutive columns of one row.
constexpr int kEpiRowPitch = 4 * 32 + 8;
template <int EPI, int TI, int TJ>
__device__ __forceinline__ void epi_wave(const v16f (&acc)[TI][TJ], float* et, int64_t mb, int64_t nb,
                                         const GemmArgs& g, int lane) {
  static_assert(TJ * 32 + 8 <= kEpiRowPitch, "row block wider than the staging pitch");
  const int r = lane & 31, c = lane >> 5;
  auto fence = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  constexpr bool kRes = EPI == kEpiResidual || EPI == kEpiBiasResidual;
  constexpr bool kBias = EPI == kEpiBias || EPI == kEpiBiasResidual || EPI == kEpiBiasGelu;
  if constexpr (EPI == kEpiBiasGeluFp4) {
    // a whole row block (32 rows x 32*TJ columns) in LDS; lane l takes row
    // l % 32 and the 16-column blocks 2q + l / 32, q < TJ, whose bias it
    // loads once as two 16-byte vectors (N % 16 == 0: a block is all in or
    // all out of range)
    const int half = lane >> 5;
    const float alpha = g.alpha, gs = g.gs_out ? *g.gs_out : 1.0f;
    u32x4 bz[TJ][2];
#pragma unroll
    for (int q = 0; q < TJ; q++) {
      const int64_t n = nb + (2 * q + half) * 16;
      const u32x4 z4 = {0u, 0u, 0u, 0u};
      bz[q][0] = n < g.N ? *reinterpret_cast<const u32x4*>(g.bias + n) : z4;
      bz[q][1] = n < g.N ? *reinterpret_cast<const u32x4*>(g.bias + n + 8) : z4;
    }
#pragma unroll
    for (int i = 0; i < TI; i++) {
#pragma unroll
      for (int j = 0; j < TJ; j++)
#pragma unroll
        for (int k = 0; k < 16; k++)
          et[((k >> 2) * 8 + c * 4 + (k & 3)) * kEpiRowPitch + j * 32 + r] = acc[i][j][k];
      fence();
      const int64_t m = mb + i * 32 + r;
#pragma unroll
      for (int q = 0; q < TJ; q++) {
        const int col = (2 * q + half) * 16;
        const int64_t n = nb + col;
        if (m < g.M && n < g.N) {
          float z[16];
#pragma unroll
          for (int v = 0; v < 4; v++) {
            const float4 tv = *reinterpret_cast<const float4*>(et + r * kEpiRowPitch + col + 4 * v);
            const uint32_t b0 = bz[q][v >> 1][2 * (v & 1)], b1 = bz[q][v >> 1][2 * (v & 1) + 1];
            z[4 * v + 0] = alpha * tv.x + bf16_lo(b0);
            z[4 * v + 1] = alpha * tv.y + bf16_hi(b0);
            z[4 * v + 2] = alpha * tv.z + bf16_lo(b1);
            z[4 * v + 3] = alpha * tv.w + bf16_hi(b1);
          }
          gelu_fp4_block(z, m, n, g, gs);
        }
      }
      fence();
    }
    return;
  }
  if (EPI == kEpiFp8 || (g.N % 8) != 0) {   // FP8 out and ragged N: tile by tile
    const int er = lane & 31, ec = (lane >> 5) * 16;
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
      for (int j = 0; j < TJ; j++) {
#pragma unroll
        for (int k = 0; k < 16; k++) et[((k >> 2) * 8 + c * 4 + (k & 3)) * kEpiPitch + r] = acc[i][j][k];
        fence();
        epi_run16<EPI>(et + er * kEpiPitch + ec, mb + i * 32 + er, nb + j * 32 + ec, g);
        fence();
      }
    return;
  }
  if constexpr (EPI != kEpiBiasGeluFp4 && EPI != kEpiFp8) {
    constexpr int kQ = 32 / 4;   // row groups of 4 per row block
    const int cl = (lane & 15) * 8, rl = lane >> 4;
    const int64_t n = nb + cl;
    const bool col_ok = cl < TJ * 32 && n < g.N;   // TJ < 4: the last lanes have no column
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    float bf[8];   // the lane's 8 bias values (zero without bias)
    {
      const u32x4 bw = (kBias && col_ok) ? *reinterpret_cast<const u32x4*>(g.bias + n) : z4;
#pragma unroll
      for (int k = 0; k < 4; k++) { bf[2 * k] = bf16_lo(bw[k]); bf[2 * k + 1] = bf16_hi(bw[k]); }
    }
    // element (mb + 32i + 4q + rl, nb + cl): a wave-uniform row-group base
    // plus the lane's 32-bit offset rl * N + cl (the row block is < 2^31 elements)
    const uint32_t loff = (uint32_t)(rl * g.N + cl);
    const float alpha = g.alpha;
    u32x4 rv[2][kQ];
    auto load_res = [&](int i, int buf) {
#pragma unroll
      for (int q = 0; q < kQ; q++) {
        const int64_t m = mb + i * 32 + q * 4 + rl;
        const uint16_t* base = g.residual + (mb + i * 32 + q * 4) * g.N + nb;
        rv[buf][q] = (kRes && col_ok && m < g.M) ? *reinterpret_cast<const u32x4*>(base + loff) : z4;
      }
    };
    if constexpr (kRes) load_res(0, 0);
#pragma unroll
    for (int i = 0; i < TI; i++) {
      if constexpr (kRes)
        if (i + 1 < TI) load_res(i + 1, (i + 1) & 1);
#pragma unroll
      for (int j = 0; j < TJ; j++)
#pragma unroll
        for (int k = 0; k < 16; k++)
          et[((k >> 2) * 8 + c * 4 + (k & 3)) * kEpiRowPitch + j * 32 + r] = acc[i][j][k];
      fence();
#pragma unroll
      for (int q = 0; q < kQ; q++) {
        const int row = q * 4 + rl;
        const int64_t m = mb + i * 32 + row;
        const float4 t0 = *reinterpret_cast<const float4*>(et + row * kEpiRowPitch + cl);
        const float4 t1 = *reinterpret_cast<const float4*>(et + row * kEpiRowPitch + cl + 4);
        const float t[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
        float z[8];
#pragma unroll
        for (int k = 0; k < 8; k++) z[k] = kBias ? __fmaf_rn(alpha, t[k], bf[k]) : alpha * t[k];
        if constexpr (kRes) {
#pragma unroll
          for (int k = 0; k < 4; k++) {
            z[2 * k] += bf16_lo(rv[i & 1][q][k]);
            z[2 * k + 1] += bf16_hi(rv[i & 1][q][k]);
          }
        }
        if constexpr (EPI == kEpiBiasGelu) {
#pragma unroll
          for (int k = 0; k < 8; k++) z[k] = gelu_erf(z[k]);
        }
        if (col_ok && m < g.M) {
          const u32x4 o = {pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]), pack_bf16x2(z[4], z[5]),
                           pack_bf16x2(z[6], z[7])};
          // nontemporal: written once, not read back by this kernel (MXFP4
          // (8192, 14336, 4096) + bias + residual: 370.6 -> 361.6 us)
          uint16_t* base = g.out + (mb + i * 32 + q * 4) * g.N + nb;
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(base + loff));
        }
      }
      fence();
    }
  }
}

// ===========================================================================
// Prefill schedule
// ===========================================================================
// 256 x 256 macro tile, 4 waves of 128 x 128 (16 accumulator tiles of 32 x 32
// per wave, 256 accumulator registers), one workgroup per CU.  A superstep's
// A and B rows (512 rows x 128 bytes = 64 KiB) are copied HBM -> LDS by the
// buffer-load-to-LDS path (no VGPR staging); two LDS buffers double-buffer
// the K loop.  Out-of-range rows and the K tail are fetched with an
// out-of-range buffer offset, which the hardware returns as zeros.
// At 128 x 128 per wave the fragment reads need 64 B/clk/CU of LDS bandwidth
// at the full MFMA rate, plus 32 B/clk for the stage writes: within the
// 128 B/clk the CU delivers.
constexpr int kPBM = 256, kPBN = 256, kPWM = 2, kPWN = 2;
constexpr int kPThreads = kPWM * kPWN * 64;
constexpr int kPStage = (kPBM + kPBN) * kSSBytes;         // 64 KiB per LDS buffer
constexpr int kPUnits = (kPBM + kPBN) * kSSBytes / 16;    // 16-byte units per stage
constexpr int kPLoads = kPUnits / kPThreads;              // 16 per thread per superstep

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16-byte chunk position of (row, chunk) in an LDS stage: rows of 128 bytes,
// chunk index XOR-ed with a row function so that the 32 rows read by one
// fragment load spread over all banks (8- and 16-lane groups alike).
__device__ __forceinline__ int lds_off(int row, int chunk) {
  const int f = (row & 7) ^ ((row >> 3) & 1);
  return row * kSSBytes + ((chunk ^ f) << 4);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int FMT, int EPI>
__global__ __launch_bounds__(kPThreads, 1) void gemm_prefill_v2_kernel(GemmArgs g) {
  constexpr int TI = kPBM / kPWM / 32, TJ = kPBN / kPWN / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kPStage];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, c = lane >> 5;
  const int wm = wave / kPWN, wn = wave % kPWN;

  // tile mapping: consecutive tiles on one XCD (workgroups are dealt to the 8
  // XCDs round-robin), then a grouped raster of 8 tile-rows
  const int64_t tiles_m = (g.M + kPBM - 1) / kPBM, tiles_n = (g.N + kPBN - 1) / kPBN;
  const int64_t T = tiles_m * tiles_n;
  int64_t t = blockIdx.x;
  if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
  const int64_t group = 8 * tiles_n;
  const int64_t first_m = (t / group) * 8;
  const int64_t gsz = (tiles_m - first_m) < 8 ? (tiles_m - first_m) : 8;
  const int64_t tm = first_m + (t % group) % gsz;
  const int64_t tn = (t % group) / gsz;
  const int64_t m0 = tm * kPBM, n0 = tn * kPBN;

  const int64_t kbytes = row_bytes<FMT>(g.K);
  const int64_t nblk = g.K / FmtTraits<FMT>::B;
  const int64_t nss = (g.K + ss_elems<FMT>() - 1) / ss_elems<FMT>();
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)(g.M * kbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.b, (short)0, (int)(g.N * kbytes), 0x00020000);

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) acc[i][j] = v16f{};

  SfWord<FMT> sa[TI], sb[TJ], sa_n[TI], sb_n[TJ];

  // Global -> LDS copy of superstep ss into buffer buf.  Unit u = i*256 + tid
  // lands at byte 16u of the stage (the DMA writes lane l of a wave at base +
  // 16 l); unit u is position u%8 of row u/8 and holds global chunk
  // (u%8) ^ f(row).  Absent rows get a base offset past the end of the
  // buffer, and chunks past K an offset past the end too, so both read as 0.
  constexpr int kAbsent = 0x40000000;   // > any operand buffer (checked by the host)
  int base_off[kPLoads];
  int chunk_off[kPLoads];
#pragma unroll
  for (int i = 0; i < kPLoads; i++) {
    const int u = i * kPThreads + tid;
    const int row = u >> 3;
    const int f = (row & 7) ^ ((row >> 3) & 1);
    chunk_off[i] = ((u & 7) ^ f) * 16;
    const int64_t gr = (i < kPLoads / 2) ? m0 + row : n0 + row - kPBM;
    const int64_t R = (i < kPLoads / 2) ? g.M : g.N;
    base_off[i] = (gr < R) ? (int)(gr * kbytes) + chunk_off[i] : kAbsent;
  }
  auto gload = [&](int64_t ss, int buf) {
    const int so = (int)(ss * kSSBytes);
#pragma unroll
    for (int i = 0; i < kPLoads; i++) {
      const int voff = (so + chunk_off[i] + 16 <= (int)kbytes) ? base_off[i] + so : kAbsent;
      lds_ptr_t dst = (lds_ptr_t)(smem + buf * kPStage + (i * kPThreads + wave * 64) * 16);
      if (i < kPLoads / 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 16, voff, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, dst, 16, voff, 0, 0, 0);
    }
  };
  auto sload = [&](int64_t ss, SfWord<FMT> (&xa)[TI], SfWord<FMT> (&xb)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; i++)
      load_sf<FMT>(xa[i], g.sfa, g.la, m0 + wm * TI * 32 + i * 32 + r, g.M, nblk, ss, c);
#pragma unroll
    for (int j = 0; j < TJ; j++)
      load_sf<FMT>(xb[j], g.sfb, g.lb, n0 + wn * TJ * 32 + j * 32 + r, g.N, nblk, ss, c);
  };
  // fragment quarter q (bytes 16q..16q+15 of each lane's 64) of buffer buf
  auto frags = [&](int buf, int q, u32x4 (&qa)[TI], u32x4 (&qb)[TJ]) {
    const uint8_t* base = smem + buf * kPStage;
#pragma unroll
    for (int i = 0; i < TI; i++)
      qa[i] = *reinterpret_cast<const u32x4*>(base + lds_off(wm * TI * 32 + i * 32 + r, quarter_off(q, c) >> 4));
#pragma unroll
    for (int j = 0; j < TJ; j++)
      qb[j] = *reinterpret_cast<const u32x4*>(
          base + lds_off(kPBM + wn * TJ * 32 + j * 32 + r, quarter_off(q, c) >> 4));
  };
  // interleave the next quarter's LDS reads with this quarter's MFMAs
  auto interleave = [&]() {
    if constexpr (FMT == kMXFP4) {
#pragma unroll
      for (int k = 0; k < TI + TJ; k++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - (TI + TJ), 0);
    }
  };

  if (nss > 0) {
    u32x4 qa[TI], qb[TJ], na[TI], nb[TJ];
    gload(0, 0);
    sload(0, sa, sb);
    wait_vm_all();
    __syncthreads();
    frags(0, 0, qa, qb);
    for (int64_t ss = 0; ss < nss; ss++) {
      const int buf = (int)(ss & 1);
      // superstep ss+1 streams into the other buffer while ss is multiplied
      // (past the end of K it reads zeros into a buffer nobody reads)
      gload(ss + 1, buf ^ 1);
      sload(ss + 1 < nss ? ss + 1 : ss, sa_n, sb_n);
      __builtin_amdgcn_sched_barrier(0);
      frags(buf, 1, na, nb);
      quarter_mma<FMT, 0, TI, TJ>(acc, qa, qb, sa, sb);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      frags(buf, 2, qa, qb);
      quarter_mma<FMT, 1, TI, TJ>(acc, na, nb, sa, sb);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      frags(buf, 3, na, nb);
      quarter_mma<FMT, 2, TI, TJ>(acc, qa, qb, sa, sb);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      // every wave has read all of buffer buf; superstep ss+1 must have landed
      wait_vm_all();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      frags(buf ^ 1, 0, qa, qb);
      quarter_mma<FMT, 3, TI, TJ>(acc, na, nb, sa, sb);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TI; i++) sa[i] = sa_n[i];
#pragma unroll
      for (int j = 0; j < TJ; j++) sb[j] = sb_n[j];
    }
    // the last gload wrote zeros into the other buffer; it lands before the
    // LDS is reused by the epilogue
    wait_vm_all();
    __syncthreads();
  }

  // epilogue: each wave stages its 32x32 tiles through its own LDS slice;
  // LDS instructions of one wave execute in order, so a wave-level barrier
  // (no workgroup barrier) orders the writes before the reads
  float* et = reinterpret_cast<float*>(smem) + wave * 32 * kEpiPitch;
  const int er = lane & 31, ec = (lane >> 5) * 16;
#pragma unroll
  for (int i = 0; i < TI; i++) {
#pragma unroll
    for (int j = 0; j < TJ; j++) {
#pragma unroll
      for (int k = 0; k < 16; k++) et[((k >> 2) * 8 + c * 4 + (k & 3)) * kEpiPitch + r] = acc[i][j][k];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      epi_run16<EPI>(et + er * kEpiPitch + ec, m0 + wm * TI * 32 + i * 32 + er,
                     n0 + wn * TJ * 32 + j * 32 + ec, g);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  if constexpr (EPI == kEpiBiasGeluFp4)
    fp4_out_padding(g, m0, m0 + kPBM, n0 / 16, (n0 + kPBN) / 16, n0 + kPBN >= g.N, tid, kPThreads);
  if constexpr (EPI == kEpiFp8)
    fp8_out_padding(g, m0, m0 + kPBM, n0 / 32, (n0 + kPBN) / 32, n0 + kPBN >= g.N, tid, kPThreads);
}

// s_waitcnt: vmcnt <= N (N < 64), lgkmcnt 0
template <int N>
__device__ __forceinline__ void wait_vm_le_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// ---------------------------------------------------------------------------
// Prefill schedule with 128-byte stages.  A stage is one 256-element
// superstep: 128 bytes of each of the 256 A and 256 B rows (64 KiB), in a
// ring of two, so every DMA instruction moves 8 whole 128-byte row segments
// (the L2 streams those at about twice the rate of 64-byte segments).  In LDS
// a row's eight 16-byte chunks are XOR-ed with (row / 2) % 8: the 16 lanes of
// one ds_read_b128 phase (rows r..r+15, one chunk each) then hit 16 distinct
// 16-byte bank groups.  One barrier per superstep, before its last quarter:
// after it the slot just consumed is refilled with superstep ss + 2 while the
// last quarter runs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int w_swz(int row) { return (row >> 1) & 7; }
// tile columns (MXFP4 and MXFP8 operands; NVFP4 runs the 128 x 384 schedule
// or, for K % 64 != 0, the 64-byte-stage one)
template <int FMT> struct PrefillTileN {
  static_assert(FMT != kNVFP4, "NVFP4 prefill runs other schedules");
  static constexpr int kCols = 256;
};
__device__ __forceinline__ int w_off(int row, int chunk) { return row * kSSBytes + ((chunk ^ w_swz(row)) << 4); }

// MXFP8 (LINEAR scales, K % 128 == 0): a superstep is 128 FP8 elements of a
// row, two scaled FP8 MFMA steps (step_f8).  SPLIT (MXFP8): workgroup (tile, y)
// runs supersteps [y * g.per, (y + 1) * g.per) with B as the MFMA row operand
// and writes its fp32 partial tiles to the workspace in the reduce pass's
// layout: tile (y, n / 32, m / 32) at ((y * ceil(N / 32) + n / 32) * ceil(M / 32)
// + m / 32) * 1024 floats, lane (r, c) holding row r and columns
// 8(k / 4) + 4c + k % 4.
template <int FMT, int EPI, bool LA_TILED, bool LB_TILED, bool SPLIT = false, bool DQ = false>
__global__ __launch_bounds__(kPThreads, 1) void gemm_prefill_w_kernel(GemmArgs g) {
  constexpr bool F8 = FMT == kMXFP8;
  static_assert(!DQ || F8, "the exact bf16 form is MXFP8's");
  static_assert(!F8 || (!LA_TILED && !LB_TILED), "MXFP8 operands take LINEAR scales");
  static_assert(!SPLIT || F8, "the split form is built for MXFP8");
  constexpr int BN = PrefillTileN<FMT>::kCols;
  constexpr int TI = kPBM / kPWM / 32, TJ = BN / kPWN / 32;
  constexpr int kStage = (kPBM + BN) * kSSBytes;            // bytes of one superstep in LDS
  constexpr int kLoadsA = kPBM * kSSBytes / 16 / kPThreads;  // 16-byte DMAs per thread: A rows
  constexpr int kLoadsAB = kStage / 16 / kPThreads;            // ... A and B rows
  // scale bytes of a row and superstep: MXFP4 8 blocks, MXFP8 4 (in the
  // TILED layout one 256-byte group per 32 rows and 8 blocks)
  constexpr int SFR = F8 ? 4 : 8;
  constexpr int SFA = kPBM * SFR, SFB = SFA + BN * SFR;
  constexpr int SFLA = SFA / 4 / kPThreads, SFL = SFB / 4 / kPThreads;   // dword DMAs per thread
  static_assert(SFB % (4 * kPThreads) == 0 && kStage % (16 * kPThreads) == 0 && kLoadsAB <= kPLoads, "DMA split");
  // outstanding DMA instructions of one stage with its scales
  constexpr int kInFlight1 = kLoadsAB + SFL;
  // the ring, the scale slots, and 256 bytes where the L2 prefetch lands
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage + 2 * SFB + 256];
  uint8_t* const sf_lds = smem + 2 * kStage;
  uint8_t* const pf_lds = sf_lds + 2 * SFB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets stay scalar
  const int r = lane & 31, c = lane >> 5;
  const int wm = wave / kPWN, wn = wave % kPWN;

  const int64_t tiles_m = (g.M + kPBM - 1) / kPBM, tiles_n = (g.N + BN - 1) / BN;
  const int64_t T = tiles_m * tiles_n;
  int64_t t = blockIdx.x;
  if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
  const int64_t group = 8 * tiles_n;
  const int64_t first_m = (t / group) * 8;
  const int64_t gsz = (tiles_m - first_m) < 8 ? (tiles_m - first_m) : 8;
  const int64_t tm = first_m + (t % group) % gsz;
  const int64_t tn = (t % group) / gsz;
  const int m0 = (int)(tm * kPBM), n0 = (int)(tn * BN);

  const int kbytes = (int)(F8 ? g.K : g.K / 2);               // bytes of a packed row
  const int nblk = (int)(g.K / 32);
  const int ktiles = (nblk + 7) >> 3;
  const int nss = (kbytes + kSSBytes - 1) / kSSBytes;          // supersteps of 128 row bytes
  // this workgroup's supersteps [s0, send) and the row bytes they cover
  const int s0 = SPLIT ? (int)blockIdx.y * g.per : 0;
  const int send = SPLIT ? min(nss, s0 + g.per) : nss;
  const int kend = min(kbytes, send * kSSBytes);
  const int M = (int)g.M, N = (int)g.N;
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, M * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.b, (short)0, N * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rssa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.sfa, (short)0, (int)sf_bytes_of(g.la, g.M, nblk), 0x00020000);
  const __amdgpu_buffer_rsrc_t rssb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.sfb, (short)0, (int)sf_bytes_of(g.lb, g.N, nblk), 0x00020000);
  constexpr int kAbsent = 0x40000000;  // beyond every operand buffer (checked by the host)

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) acc[i][j] = v16f{};

  // per-thread DMA geometry of a stage (one superstep, 128 bytes per row):
  // unit u = i*256 + tid is position u%8 of row u/8 and fetches global chunk
  // (u%8) ^ f(row), so the 8 lanes of a row move its 128 bytes in one request
  // sized for the widest tile (kPLoads >= kLoadsAB): an array whose bound is
  // the width-dependent constant, captured by the lambdas below, drops the
  // kernel's host-side instantiation
  int base_off[kPLoads], chunk_off[kPLoads];
#pragma unroll
  for (int i = 0; i < kLoadsAB; i++) {
    const int u = i * kPThreads + tid;
    const int row = u >> 3;
    chunk_off[i] = ((u & 7) ^ w_swz(row)) * 16;
    const int gr = (i < kLoadsA) ? m0 + row : n0 + row - kPBM;
    const int R = (i < kLoadsA) ? M : N;
    base_off[i] = (gr < R) ? gr * kbytes + chunk_off[i] : kAbsent;
  }
  // L2 prefetch of a later superstep: lane l of wave w touches the 128-byte
  // segment of A row m0 + 64w + l and of B row n0 + 64w + l (one dword each,
  // written to a throwaway LDS word, so no register waits for it)
  constexpr int kPf = 2;   // prefetch instructions per wave per superstep
  const int pf_a = (m0 + wave * 64 + lane < M) ? (m0 + wave * 64 + lane) * kbytes : kAbsent;
  const int pf_b = (wave * 64 + lane < BN && n0 + wave * 64 + lane < N) ? (n0 + wave * 64 + lane) * kbytes : kAbsent;
  // Past the last superstep the instruction still goes out (the wait counts
  // assume kPf of them) but with the out-of-range lane offset: only that one
  // is range-checked, and the superstep's advance in the scalar offset would
  // otherwise reach past the end of the buffer on its last row.
  auto prefetch = [&](int k) {
    const bool ok = k < send;   // uniform
    const int so = ok ? k * kSSBytes : 0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)pf_lds, 4, ok ? pf_a : kAbsent, so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)pf_lds, 4, ok ? pf_b : kAbsent, so, 0, 0);
  };

  // superstep k -> ring slot k % 2 (and, with_sf, its scales -> scale slot
  // k % 2), masked at the K tail and past M / N.  Branch-free, so that the
  // whole loop body is one basic block the scheduler keeps in the written order.
  constexpr bool la_t = LA_TILED, lb_t = LB_TILED;
  auto issue = [&](int k, auto with_sf) {
    const int so = k * kSSBytes;
    uint8_t* slot = smem + (k & 1) * kStage;
#pragma unroll
    for (int i = 0; i < kLoadsAB; i++) {
      const int voff = (so + chunk_off[i] + 16 <= kend) ? base_off[i] + so : kAbsent;
      lds_ptr_t dst = (lds_ptr_t)(slot + (i * kPThreads + wave * 64) * 16);
      if (i < kLoadsA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 16, voff, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, dst, 16, voff, 0, 0, 0);
    }
    if constexpr (decltype(with_sf)::value) {
      const int ss = k;
      uint8_t* sfs = sf_lds + (ss & 1) * SFB;
#pragma unroll
      for (int q = 0; q < SFL; q++) {
        const bool is_a = q < SFLA;              // the first SFLA dwords: A (uniform)
        const int dd = (is_a ? q : q - SFLA) * kPThreads + tid;
        const int row0 = is_a ? m0 : n0, R = is_a ? M : N;
        const bool tiled = is_a ? la_t : lb_t;   // compile-time per q
        int vt, vl;
        bool okt, okl;
        if constexpr (F8) {   // LINEAR: one word (4 blocks) of a row per superstep
          const int gr = row0 + dd;
          okt = false;
          vt = 0;
          okl = ss < send && gr < R;
          vl = gr * nblk + 4 * ss;
        } else {   // MXFP4: two words (8 blocks) of a row, or a 256-byte TILED group per 32 rows
          const int grp = (row0 >> 5) + (dd >> 6);
          okt = ss < nss && grp * 32 < R;
          vt = ((grp * ktiles + ss) << 8) + ((dd & 63) << 2);
          const int gr = row0 + (dd >> 1);
          okl = ss < nss && gr < R;
          vl = gr * nblk + 8 * ss + 4 * (dd & 1);
        }
        const int voff = tiled ? (okt ? vt : kAbsent) : (okl ? vl : kAbsent);
        lds_ptr_t dst = (lds_ptr_t)(sfs + (q * kPThreads + wave * 64) * 4);
        if (is_a)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rssa, dst, 4, voff, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rssb, dst, 4, voff, 0, 0, 0);
      }
    }
  };
  using kWithSf = std::integral_constant<bool, true>;

  // Steady state: when stage k and the scales of superstep k/2 lie wholly
  // inside K, a lane's DMA offsets do not depend on k; the per-stage advance
  // goes into the scalar offset and the LDS targets are scalar, so a DMA is
  // one s_mov to m0 and one buffer_load (rows past M / N keep kAbsent).
  int sf_voff[SFL];
#pragma unroll
  for (int q = 0; q < SFL; q++) {
    const bool is_a = q < SFLA;
    const int dd = (is_a ? q : q - SFLA) * kPThreads + tid;
    const int row0 = is_a ? m0 : n0, R = is_a ? M : N;
    const bool tiled = is_a ? la_t : lb_t;
    if constexpr (F8) {
      const int gr = row0 + dd;
      sf_voff[q] = gr < R ? gr * nblk : kAbsent;
    } else {
      const int grp = (row0 >> 5) + (dd >> 6);
      const int gr = row0 + (dd >> 1);
      sf_voff[q] = tiled ? (grp * 32 < R ? ((grp * ktiles) << 8) + ((dd & 63) << 2) : kAbsent)
                         : (gr < R ? gr * nblk + 4 * (dd & 1) : kAbsent);
    }
  }
  auto issue_fast = [&](int k, auto with_sf) {
    const int so = k * kSSBytes;
    uint8_t* slot = smem + (k & 1) * kStage;
#pragma unroll
    for (int i = 0; i < kLoadsAB; i++) {
      lds_ptr_t dst = (lds_ptr_t)(slot + (i * kPThreads + wave * 64) * 16);
      if (i < kLoadsA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 16, base_off[i], so, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, dst, 16, base_off[i], so, 0, 0);
    }
    if constexpr (decltype(with_sf)::value) {
      const int ss = k;
      uint8_t* sfs = sf_lds + (ss & 1) * SFB;
      // scalar advance per superstep: one 256-byte group column in the tiled
      // layout, 8 (MXFP4) or 4 (MXFP8) bytes of a row in the linear one
      const int adv_t = ss << 8;
      const int adv_l = F8 ? (ss << 2) : (ss << 3);
      const int soa = la_t ? adv_t : adv_l, sob = lb_t ? adv_t : adv_l;
#pragma unroll
      for (int q = 0; q < SFL; q++) {
        lds_ptr_t dst = (lds_ptr_t)(sfs + (q * kPThreads + wave * 64) * 4);
        if (q < SFLA)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rssa, dst, 4, sf_voff[q], soa, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rssb, dst, 4, sf_voff[q], sob, 0, 0);
      }
    }
  };

  // the lane's scale words of superstep ss from its LDS area, branch-free:
  // two dwords are read and v_perm picks the lane's four bytes
  auto read_sf = [&](int ss, SfWord<FMT> (&xa)[TI], SfWord<FMT> (&xb)[TJ], auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const uint8_t* sfs = sf_lds + (ss & 1) * SFB;
    const int left = nblk - ss * 8;   // MXFP4 blocks of this superstep that exist
#pragma unroll
    for (int side = 0; side < 2; side++) {
      const bool tiled = side ? lb_t : la_t;
      const uint8_t* area = sfs + side * SFA;
#pragma unroll
      for (int i = 0; i < (side ? TJ : TI); i++) {
        const int grp = (side ? wn * TJ : wm * TI) + i;     // 32-row group inside the tile
        const int row = grp * 32 + r;
        SfWord<FMT>& o = side ? xb[i] : xa[i];
        if constexpr (F8) {
          // blocks 4ss .. 4ss + 3 of the row; lane half c takes block 2Q + c
          // in step Q, found at byte 2Q once the word is shifted by 8c
          // (every superstep is whole: K % 128 == 0)
          o.w = *reinterpret_cast<const uint32_t*>(area + row * 4) >> (DQ ? 0 : 8 * c);
          (void)tiled;
        } else {
          const int a0 = tiled ? grp * 256 + (c * 32 + r) * 4 : row * 8;
          const uint32_t lo = *reinterpret_cast<const uint32_t*>(area + a0);
          uint32_t w = lo;    // tiled: the word is the lane's four blocks
          if (!tiled) w = __builtin_amdgcn_perm(*reinterpret_cast<const uint32_t*>(area + a0 + 4), lo, pair_sel(c));
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const bool absent = MASK && 2 * c + (j & 1) + 4 * (j >> 1) >= left;
            w = absent ? (w & ~(0xFFu << (8 * j))) | (0x7Fu << (8 * j)) : w;
          }
          o.w = w;
        }
      }
    }
  };

  // quarter Q of superstep k: the lane's 16 bytes at 64(Q/2) + 32c + 16(Q%2)
  // of each 128-byte row; MXFP8 at 64(Q/2) + 16c + 32(Q%2) (step_f8)
  auto frags = [&](int k, int s, u32x4 (&qa)[TI], u32x4 (&qb)[TJ]) {
    const uint8_t* base = smem + (k & 1) * kStage;
    const int ch = F8 ? 4 * (s >> 1) + c + 2 * (s & 1) : 4 * (s >> 1) + 2 * c + (s & 1);
    // order of first use by quarter_mma (i outer, j inner): a0, b0..b3, a1..a3
    qa[0] = *reinterpret_cast<const u32x4*>(base + w_off(wm * TI * 32 + r, ch));
#pragma unroll
    for (int j = 0; j < TJ; j++)
      qb[j] = *reinterpret_cast<const u32x4*>(base + w_off(kPBM + wn * TJ * 32 + j * 32 + r, ch));
#pragma unroll
    for (int i = 1; i < TI; i++)
      qa[i] = *reinterpret_cast<const u32x4*>(base + w_off(wm * TI * 32 + i * 32 + r, ch));
  };
  // MXFP4: after each of the first TI + TJ MFMAs of a quarter DSR next-quarter
  // LDS reads, then after each of the following MFMAs DMAs until VM are
  // issued.  The reads come first: the compiler cannot tell the DMA's LDS
  // writes (another ring slot) from the reads, so it keeps them in that order.
  auto interleave = [&](auto dsr, auto vm) {
    constexpr int DSR = decltype(dsr)::value, VM = decltype(vm)::value;
    if constexpr (FMT == kMXFP4 || F8) {
      constexpr int NR = TI + TJ;                              // MFMAs carrying reads
      constexpr int NV = TI * TJ - NR;                         // MFMAs that can carry DMAs
      constexpr int PER = (VM + NV - 1) / (NV > 0 ? NV : 1);   // DMAs per such MFMA
#pragma unroll
      for (int k = 0; k < TI * TJ; k++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if (k < NR) {
          __builtin_amdgcn_sched_group_barrier(0x100, DSR, 0);   // LDS reads
        } else if (VM > 0 && (k - NR) * PER < VM) {
          __builtin_amdgcn_sched_group_barrier(0x010, PER, 0);   // DMAs
        }
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using ILSP = std::integral_constant<int, kLoadsAB + SFL + kPf>;
  // VM: DMA instructions issued after the stage being waited for (the prefetch)
  auto stage_barrier = [&](auto vm) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_le_lgkm0<decltype(vm)::value>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  SfWord<FMT> sa[TI], sb[TJ], sa_n[TI], sb_n[TJ];
  u32x4 qa[TI], qb[TJ], na[TI], nb[TJ];
  u32x4 qa2[TI], qb2[TJ], na2[TI], nb2[TJ];   // MXFP8: quarters 2 and 3 (step 1)
  issue(s0, kWithSf{});
  issue(s0 + 1, kWithSf{});
  prefetch(s0 + 2);   // every stage is followed by kPf prefetch instructions
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_le_lgkm0<kInFlight1 + kPf>();   // superstep s0 has landed (s0 + 1 may be in flight)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_sf(s0, sa, sb, std::true_type{});
  frags(s0, 0, qa, qb);
  if constexpr (F8 && !DQ) frags(s0, 1, na, nb);
  // supersteps whose refill (superstep ss + 2, scales included) lies wholly
  // inside this workgroup's K: ss + 2 < min(send, whole supersteps of K)
  const int nfast = max(s0, min(send, kbytes / kSSBytes) - 2);
  // superstep ss from slot ss % 2: quarters 0-2, then one barrier (superstep
  // ss + 1 has landed; every wave is done with slot ss % 2, whose last
  // quarter is already in registers), then quarter 3 reads superstep ss + 1
  // and refills slot ss % 2 with superstep ss + 2
  using I3 = std::integral_constant<int, 3>;
  // MXFP8: on entry (qa, qb) and (na, nb) hold quarters 0 and 1 of superstep
  // ss; step 0 runs on them while quarters 2 and 3 are read, then (after the
  // barrier) step 1 runs on those while the next superstep's quarters 0 and 1
  // and its scale words are read and slot ss % 2 is refilled
  auto superstep_f8 = [&](int ss, auto fast) {
    constexpr bool F = decltype(fast)::value;
    frags(ss, 2, qa2, qb2);
    frags(ss, 3, na2, nb2);
    step_f8<0, SPLIT>(acc, qa, na, qb, nb, sa, sb);
    interleave(I2{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    if (F || ss == nfast) stage_barrier(std::integral_constant<int, kPf>{});
    else stage_barrier(std::integral_constant<int, 0>{});
    if constexpr (F) {
      read_sf(ss + 1, sa_n, sb_n, std::false_type{});
      frags(ss + 1, 0, qa, qb);
      frags(ss + 1, 1, na, nb);
      issue_fast(ss + 2, kWithSf{});
      prefetch(ss + 3);
    } else {
      issue(ss + 2, kWithSf{});
      __builtin_amdgcn_sched_barrier(0);
      read_sf(ss + 1, sa_n, sb_n, std::false_type{});
      frags(ss + 1, 0, qa, qb);
      frags(ss + 1, 1, na, nb);
    }
    step_f8<1, SPLIT>(acc, qa2, na2, qb2, nb2, sa, sb);
    if constexpr (F) interleave(I3{}, ILSP{}); else interleave(I3{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TI; i++) sa[i] = sa_n[i];
#pragma unroll
    for (int j = 0; j < TJ; j++) sb[j] = sb_n[j];
  };
  auto superstep = [&](int ss, auto fast) {
    constexpr bool F = decltype(fast)::value;
    frags(ss, 1, na, nb);
    if constexpr (DQ) quarter_f8dq<0, SPLIT>(acc, qa, qb, sa, sb);
    else quarter_mma<FMT, 0, TI, TJ>(acc, qa, qb, sa, sb);
    interleave(I1{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    frags(ss, 2, qa, qb);
    if constexpr (DQ) quarter_f8dq<1, SPLIT>(acc, na, nb, sa, sb);
    else quarter_mma<FMT, 1, TI, TJ>(acc, na, nb, sa, sb);
    interleave(I1{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    frags(ss, 3, na, nb);
    if constexpr (DQ) quarter_f8dq<2, SPLIT>(acc, qa, qb, sa, sb);
    else quarter_mma<FMT, 2, TI, TJ>(acc, qa, qb, sa, sb);
    interleave(I1{}, I0{});
    // superstep ss + 1 was issued by the previous superstep (or the prologue)
    // and followed by kPf prefetch instructions when that one was a
    // steady-state superstep (the prologue always prefetches)
    if (F || ss == nfast) stage_barrier(std::integral_constant<int, kPf>{});
    else stage_barrier(std::integral_constant<int, 0>{});
    if constexpr (F) {
      read_sf(ss + 1, sa_n, sb_n, std::false_type{});
      frags(ss + 1, 0, qa, qb);
      issue_fast(ss + 2, kWithSf{});
      prefetch(ss + 3);
    } else {
      issue(ss + 2, kWithSf{});
      __builtin_amdgcn_sched_barrier(0);
      read_sf(ss + 1, sa_n, sb_n, std::true_type{});
      frags(ss + 1, 0, qa, qb);
    }
    if constexpr (DQ) quarter_f8dq<3, SPLIT>(acc, na, nb, sa, sb);
    else quarter_mma<FMT, 3, TI, TJ>(acc, na, nb, sa, sb);
    if constexpr (F) interleave(I2{}, ILSP{}); else interleave(I2{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TI; i++) sa[i] = sa_n[i];
#pragma unroll
    for (int j = 0; j < TJ; j++) sb[j] = sb_n[j];
  };
  int ss = s0;
  if constexpr (F8 && !DQ) {
    for (; ss < nfast; ss++) superstep_f8(ss, std::true_type{});
    for (; ss < send; ss++) superstep_f8(ss, std::false_type{});
  } else {
    for (; ss < nfast; ss++) superstep(ss, std::true_type{});
    for (; ss < send; ss++) superstep(ss, std::false_type{});
  }
  // the DMA issued past the end (zeros) lands before the epilogue reuses LDS
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __syncthreads();

  if constexpr (SPLIT) {
    // acc[i][j] is the transposed tile (B was the row operand): lane (r, c)
    // holds row m of A tile i and columns 8(k / 4) + 4c + k % 4 of B tile j,
    // the partial layout; tiles wholly past M or N are not part of it
    const int64_t tn32 = (g.N + 31) / 32, tm32 = (g.M + 31) / 32;
    const int64_t y = blockIdx.y;
#pragma unroll
    for (int i = 0; i < TI; i++) {
      const int64_t mt = (m0 + wm * TI * 32) / 32 + i;
#pragma unroll
      for (int j = 0; j < TJ; j++) {
        const int64_t nt = (n0 + wn * TJ * 32) / 32 + j;
        if (mt < tm32 && nt < tn32) {
          float4* p = reinterpret_cast<float4*>(g.ws + ((y * tn32 + nt) * tm32 + mt) * 1024 + lane * 16);
#pragma unroll
          for (int q = 0; q < 4; q++)
            p[q] = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
    }
    return;
  }
  epi_wave<EPI, TI, TJ>(acc, reinterpret_cast<float*>(smem) + wave * 32 * kEpiRowPitch, m0 + wm * TI * 32,
                        n0 + wn * TJ * 32, g, lane);
  if constexpr (EPI == kEpiBiasGeluFp4)
    fp4_out_padding(g, m0, m0 + kPBM, n0 / 16, (n0 + BN) / 16, n0 + BN >= g.N, tid, kPThreads);
  if constexpr (EPI == kEpiFp8)
    fp8_out_padding(g, m0, m0 + kPBM, n0 / 32, (n0 + BN) / 32, n0 + BN >= g.N, tid, kPThreads);
}

// ===========================================================================
// Decode schedule (weights as the MFMA row operand, K split across waves)
// ===========================================================================
// Decode schedule.  SPLIT: split-K -- workgroup (tile, y) takes supersteps
// [y * g.per, (y + 1) * g.per) of K and writes its partial C^T tiles, in the
// MFMA accumulator layout (lane-major, 16 floats a lane), to the workspace
// at g.ws + ((y * tiles + tile) * MT + i) * 1024; gemm_splitk_reduce_kernel
// sums the partials and applies the epilogue.
template <int FMT, int MT, int W, int EPI, bool DB = true, bool HALF = false, bool SPLIT = false>
__global__ __launch_bounds__(W * 64) void gemm_decode_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float red[W * MT * 64 * 16];
  __shared__ __attribute__((aligned(16))) float tile[SPLIT ? 1 : MT * 32 * kEpiPitch];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, c = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int64_t kbytes = row_bytes<FMT>(g.K);
  const int64_t nblk = g.K / FmtTraits<FMT>::B;
  const int64_t nss_all = (g.K + ss_elems<FMT>() - 1) / ss_elems<FMT>();
  const int64_t s_begin = SPLIT ? (int64_t)blockIdx.y * g.per : 0;
  const int64_t nss = SPLIT ? (s_begin + g.per < nss_all ? s_begin + g.per : nss_all) : nss_all;

  v16f acc[1][MT];
#pragma unroll
  for (int i = 0; i < MT; i++) acc[0][i] = v16f{};

  // DB: two supersteps in flight per wave -- the loads of superstep ss + W are
  // issued before the MFMAs of ss (buffers 0 / 1 alternate, unrolled by two
  // so that every register index stays static).  Otherwise one superstep at a
  // time, which leaves registers for twice the waves (see the launcher).
  Frag fw[2][1], fx[2][MT];
  SfWord<FMT> sw[2][1], sx[2][MT];
  auto load = [&](auto bufc, int64_t ss) {
    constexpr int buf = decltype(bufc)::value;
    Frag(&w)[1] = fw[buf];
    Frag(&x)[MT] = fx[buf];
    SfWord<FMT>(&ws)[1] = sw[buf];
    SfWord<FMT>(&xs)[MT] = sx[buf];
    load_frag_global<HALF>(w[0], g.b, n0 + r, g.N, kbytes, ss, c);
    load_sf<FMT>(ws[0], g.sfb, g.lb, n0 + r, g.N, nblk, ss, c);
#pragma unroll
    for (int i = 0; i < MT; i++) {
      load_frag_global<HALF>(x[i], g.a, 32 * i + r, g.M, kbytes, ss, c);
      load_sf<FMT>(xs[i], g.sfa, g.la, 32 * i + r, g.M, nblk, ss, c);
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int64_t ss = s_begin + wave;
  if constexpr (DB) {
    if (ss < nss) load(B0{}, ss);
    for (; ss < nss; ss += 2 * W) {
      if (ss + W < nss) load(B1{}, ss + W);
      superstep_mma<FMT, 1, MT>(acc, fw[0], fx[0], sw[0], sx[0]);
      if (ss + W >= nss) break;
      if (ss + 2 * W < nss) load(B0{}, ss + 2 * W);
      superstep_mma<FMT, 1, MT>(acc, fw[1], fx[1], sw[1], sx[1]);
    }
  } else {
    for (; ss < nss; ss += W) {
      load(B0{}, ss);
      superstep_mma<FMT, 1, MT>(acc, fw[0], fx[0], sw[0], sx[0]);
    }
  }

  // cross-wave sum of the partial C^T tiles: every wave writes its
  // accumulators, then thread t sums element e = t, t + 64 W, .. over the W
  // waves in wave order (one barrier; element e = (i * 64 + l) * 16 + k is
  // accumulator k of lane l for M-tile i)
#pragma unroll
  for (int i = 0; i < MT; i++)
#pragma unroll
    for (int k = 0; k < 16; k++) red[((wave * MT + i) * 64 + lane) * 16 + k] = acc[0][i][k];
  __syncthreads();
  if constexpr (SPLIT) {
    // the partial goes out in the accumulator layout, consecutive threads
    // writing consecutive floats
    float* dst = g.ws + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * MT * 1024;
    for (int e = tid; e < MT * 64 * 16; e += W * 64) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < W; w++) s += red[w * MT * 64 * 16 + e];
      dst[e] = s;
    }
  } else {
    for (int e = tid; e < MT * 64 * 16; e += W * 64) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < W; w++) s += red[w * MT * 64 * 16 + e];
      // C^T row n = (k/4)*8 + (l/32)*4 + k%4, column m = l % 32
      const int i = e / 1024, l = (e / 16) % 64, k = e % 16;
      const int nl = (k >> 2) * 8 + (l >> 5) * 4 + (k & 3), ml = l & 31;
      tile[(i * 32 + ml) * kEpiPitch + nl] = s;
    }
    __syncthreads();
    if (wave < MT) {
      const int er = lane & 31, ec = (lane >> 5) * 16;
      epi_run16<EPI>(tile + (wave * 32 + er) * kEpiPitch + ec, wave * 32 + er, n0 + ec, g);
    }
    if constexpr (EPI == kEpiBiasGeluFp4)
      fp4_out_padding(g, 0, (g.M + 31) / 32 * 32, n0 / 16, (n0 + 32) / 16, n0 + 32 >= g.N, tid, W * 64);
    if constexpr (EPI == kEpiFp8)
      fp8_out_padding(g, 0, 128, n0 / 32, n0 / 32 + 1, n0 + 32 >= g.N, tid, W * 64);
  }
}

// Split-K second pass: one wave per (32-column tile, M-tile): the partials
// of the g.splits workgroups are summed in split order (the result does not
// depend on timing), transposed through LDS, and the epilogue applied.
template <int EPI>
__global__ __launch_bounds__(64) void gemm_splitk_reduce_kernel(GemmArgs g, int MT) {
  __shared__ __attribute__((aligned(16))) float t[32 * kEpiPitch];
  const int lane = threadIdx.x, r = lane & 31, c = lane >> 5;
  const int64_t tiles = gridDim.x, tile = blockIdx.x, i = blockIdx.y;
  const int64_t n0 = tile * 32;
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; k++) v[k] = 0.0f;
  for (int y = 0; y < g.splits; y++) {
    const float4* p = reinterpret_cast<const float4*>(g.ws + ((y * tiles + tile) * MT + i) * 1024 + lane * 16);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float4 w = p[q];
      v[4 * q] += w.x;
      v[4 * q + 1] += w.y;
      v[4 * q + 2] += w.z;
      v[4 * q + 3] += w.w;
    }
  }
#pragma unroll
  for (int k = 0; k < 16; k++) t[r * kEpiPitch + (k >> 2) * 8 + c * 4 + (k & 3)] = v[k];
  __syncthreads();
  const int ec = c * 16;
  epi_run16<EPI>(t + r * kEpiPitch + ec, i * 32 + r, n0 + ec, g);
  if constexpr (EPI == kEpiBiasGeluFp4)
    fp4_out_padding(g, i * 32, i * 32 + 32, n0 / 16, (n0 + 32) / 16, n0 + 32 >= g.N, lane, 64);
  if constexpr (EPI == kEpiFp8)   // the last M-tile also owns the padding rows (to a multiple of 128)
    fp8_out_padding(g, i * 32, (i + 1 == MT) ? sf_pad_rows(kSwz128, g.M) : i * 32 + 32, n0 / 32, n0 / 32 + 1,
                    n0 + 32 >= g.N, lane, 64);
}

#include "gemm_nv.hpp"

template <int FMT, int EPI, bool SPLIT = false, bool DQ = false>
void launch_w(const GemmArgs& g, dim3 block, hipStream_t s) {
  constexpr int BN = PrefillTileN<FMT>::kCols;
  const dim3 grid((unsigned)(((g.M + kPBM - 1) / kPBM) * ((g.N + BN - 1) / BN)), SPLIT ? (unsigned)g.splits : 1u);
  if constexpr (FMT == kMXFP8)   // LINEAR scales only
    hipLaunchKernelGGL((gemm_prefill_w_kernel<FMT, EPI, false, false, SPLIT, DQ>), grid, block, 0, s, g);
  else if (g.la == kTiled && g.lb == kTiled)
    hipLaunchKernelGGL((gemm_prefill_w_kernel<FMT, EPI, true, true>), grid, block, 0, s, g);
  else if (g.la == kTiled)
    hipLaunchKernelGGL((gemm_prefill_w_kernel<FMT, EPI, true, false>), grid, block, 0, s, g);
  else if (g.lb == kTiled)
    hipLaunchKernelGGL((gemm_prefill_w_kernel<FMT, EPI, false, true>), grid, block, 0, s, g);
  else
    hipLaunchKernelGGL((gemm_prefill_w_kernel<FMT, EPI, false, false>), grid, block, 0, s, g);
}

// Decode launch: the workgroup size and buffering by format and M-tiles.
// NVFP4 is bound by its dequantization VALU work: 8 single-buffered waves
// (two per SIMD) beat double-buffered ones at 1, 3 and 4 M-tiles, e.g.
// (128, 17408, 5120) GELU -> FP4 87.6 -> 66.3 us, (128, 5120, 17408) 86.3
// -> 65.8 us, (1, 5120, 17408) 26.0 -> 23.4 us.  MXFP4, bound by load
// latency, keeps two supersteps in flight (its single-buffered forms
// measured 15-35% slower), as does NVFP4 at 2 M-tiles.
template <int FMT, int EPI, bool HALF>
hipError_t launch_decode(const GemmArgs& g, hipStream_t s) {
  const unsigned grid = (unsigned)((g.N + 31) / 32);
  const int mt = (int)((g.M + 31) / 32);
#define LB_DEC(MT, W, DB)                                                                               \
  if (mt == MT) {                                                                                       \
    hipLaunchKernelGGL((gemm_decode_kernel<FMT, MT, W, EPI, DB, HALF>), dim3(grid), dim3(W * 64), 0, s, g); \
    return hipGetLastError();                                                                           \
  }
  if constexpr (FMT == kNVFP4) {
    LB_DEC(1, 8, false) LB_DEC(2, 8, true) LB_DEC(3, 8, false) LB_DEC(4, 8, false)
  } else {   // MXFP4, and MXFP8 (its dequantization is half an instruction an element)
    LB_DEC(1, 8, true) LB_DEC(2, 8, true) LB_DEC(3, 4, true) LB_DEC(4, 4, true)
  }
#undef LB_DEC
  return hipErrorInvalidValue;
}

// NVFP4 with K % 32 == 16 (packed rows 8 mod 16 bytes) runs on the decode
// schedule only, whose register loads take 8-byte halves; the prefill
// schedule stages 16-byte row chunks by DMA.  More than 128 rows go as
// consecutive decode launches over 128-row slices of A (and of the residual
// and output), each slice starting on a 32-row scale group.
template <int FMT, int EPI>
hipError_t launch_decode_rows(const GemmArgs& g, hipStream_t s) {
  const bool half = FMT == kNVFP4 && (g.K / 2) % 16 != 0;
  if (g.M <= 128)
    return half ? launch_decode<FMT, EPI, FMT == kNVFP4>(g, s) : launch_decode<FMT, EPI, false>(g, s);
  const int64_t kbytes = row_bytes<FMT>(g.K), nblk = g.K / FmtTraits<FMT>::B;
  const int64_t nblk_out = g.N / (EPI == kEpiFp8 ? 32 : 16);
  for (int64_t m0 = 0; m0 < g.M; m0 += 128) {
    GemmArgs q = g;
    q.M = (g.M - m0) < 128 ? (g.M - m0) : 128;
    q.a = g.a + m0 * kbytes;
    q.sfa = g.sfa + (g.la == kTiled ? (m0 / 32) * ((nblk + 7) / 8) * 256 : m0 * nblk);
    if (g.residual) q.residual = g.residual + m0 * g.N;
    if (g.out) q.out = g.out + m0 * g.N;
    if (g.out_packed) q.out_packed = g.out_packed + m0 * (EPI == kEpiFp8 ? g.N : g.N / 2);
    // m0 is a multiple of 128: the scale bytes of rows < m0 come first in
    // every layout, whole 32-row (TILED) and 128-row (128 x 4) groups
    if (g.out_sf) q.out_sf = g.out_sf + sf_bytes_of(g.out_layout, m0, nblk_out);
    const hipError_t e =
        half ? launch_decode<FMT, EPI, FMT == kNVFP4>(q, s) : launch_decode<FMT, EPI, false>(q, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int FMT, int EPI>
hipError_t launch_fmt_epi(const GemmArgs& g, int variant, hipStream_t s) {
  if (variant == 0) return launch_decode_rows<FMT, EPI>(g, s);
  const int64_t T = ((g.M + kPBM - 1) / kPBM) * ((g.N + kPBN - 1) / kPBN);
  // MXFP8 operands on the scaled FP8 MFMA (f8mma) with K % 128 == 0 run the
  // 128-byte-stage schedule; NVFP4 (K % 64 == 0) and exact MXFP8 (K % 128
  // == 0) operands the 128 x 384 schedule (every epilogue); other NVFP4 and
  // MXFP8 operands the 64-byte-stage prefill kernel, MXFP4 the 128-byte-stage
  // one.  The 128-byte-stage and 128 x 384 kernels fetch LINEAR scales as
  // aligned words, which needs the blocks per row to be a multiple of 4 and a
  // 4-byte aligned base (else the 64-byte-stage kernel)
  if constexpr (FMT == kMXFP8) {
    if (prefill_nv_ok<FMT>(g)) {
      if (g.f8mma) launch_w<FMT, EPI>(g, dim3(kPThreads), s);
      else launch_w<FMT, EPI, false, true>(g, dim3(kPThreads), s);
      return hipGetLastError();
    }
  }
  if constexpr (FMT == kNVFP4) {
    if (prefill_nv_ok<FMT>(g)) {
      launch_prefill_nv<FMT, EPI>(g, s);
      return hipGetLastError();
    }
  }
  if constexpr (FMT == kMXFP8 || FMT == kNVFP4) {
    // (NVFP4 with K % 64 == 32 and TILED scales: 4096 x 4096 x 8224 and
    // 2048 x 8192 x 4128 ran 288-298 / 151-153 us here against 348-352 /
    // 182-184 us on the 128-byte-stage kernel)
    hipLaunchKernelGGL((gemm_prefill_v2_kernel<FMT, EPI>), dim3((unsigned)T), dim3(kPThreads), 0, s, g);
  } else {
    const int64_t nblk = g.K / FmtTraits<FMT>::B;
    auto dword_ok = [&](const uint8_t* p, int lay) {
      return lay == kTiled || (nblk % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 3) == 0);
    };
    if (dword_ok(g.sfa, g.la) && dword_ok(g.sfb, g.lb)) {
      const dim3 grid((unsigned)T), block(kPThreads);
      launch_w<FMT, EPI>(g, block, s);
    } else
      hipLaunchKernelGGL((gemm_prefill_v2_kernel<FMT, EPI>), dim3((unsigned)T), dim3(kPThreads), 0, s, g);
  }
  return hipGetLastError();
}

// Split-K launch: the partial pass (decode kernel with SPLIT; one
// instantiation per format, M-tiles, waves and half-chunk flag, shared by
// the epilogues) and the reduce pass with the epilogue.
template <int FMT, int EPI, int MT, bool HALF>
hipError_t launch_splitk_mt(const GemmArgs& g, hipStream_t s) {
  // MXFP4 and MXFP8 keep two supersteps in flight per wave, NVFP4 (bound by
  // its dequantization work) one, as in the decode schedule
  constexpr bool DB = FMT != kNVFP4;
  const unsigned tiles = (unsigned)((g.N + 31) / 32);
  const dim3 grid(tiles, (unsigned)g.splits);
  if (g.per >= 4)
    hipLaunchKernelGGL((gemm_decode_kernel<FMT, MT, 4, kEpiNone, DB, HALF, true>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_decode_kernel<FMT, MT, 2, kEpiNone, DB, HALF, true>), grid, dim3(128), 0, s, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_splitk_reduce_kernel<EPI>), dim3(tiles, (unsigned)MT), dim3(64), 0, s, g, MT);
  return hipGetLastError();
}

template <int FMT, int EPI>
hipError_t launch_splitk(const GemmArgs& g, hipStream_t s) {
  const int mt = (int)((g.M + 31) / 32);
  if constexpr (FMT == kNVFP4 || FMT == kMXFP8) {
    if (g.split_nv) {   // partials from a prefill schedule, same reduce
      if (!prefill_nv_ok<FMT>(g)) return hipErrorInvalidValue;
      if constexpr (FMT == kMXFP8) {   // 256 x 256 tiles, supersteps of 128 elements
        if (g.f8mma) launch_w<FMT, kEpiNone, true, false>(g, dim3(kPThreads), s);
        else launch_w<FMT, kEpiNone, true, true>(g, dim3(kPThreads), s);
      } else {                         // 128 x 384 tiles, stages of 64 bytes
        launch_prefill_nv<FMT, kEpiNone, true>(g, s);
      }
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gemm_splitk_reduce_kernel<EPI>), dim3((unsigned)((g.N + 31) / 32), (unsigned)mt),
                         dim3(64), 0, s, g, mt);
      return hipGetLastError();
    }
  }
  const bool half = FMT == kNVFP4 && (g.K / 2) % 16 != 0;
#define LB_SPLIT(MT)                                                                        \
  if (mt == MT)                                                                             \
    return half ? launch_splitk_mt<FMT, EPI, MT, (FMT == kNVFP4)>(g, s)                   \
                : launch_splitk_mt<FMT, EPI, MT, false>(g, s);
  LB_SPLIT(1) LB_SPLIT(2) LB_SPLIT(3) LB_SPLIT(4)
#undef LB_SPLIT
  return hipErrorInvalidValue;
}

}  // namespace gk
}  // namespace lowbit
