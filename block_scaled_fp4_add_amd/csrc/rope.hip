// rope.hip -- inverse RoPE + MX quantization of attention rows for gfx950
// (vLLM page deepseek_v41/nvidia/ops/fused_wo_a, FusedWoAKernel.device_kernel,
// its activation quant stage: bf16 rows of a head, the rotary slice rotated
// back, 32-element blocks with an MX scale and FP8 elements).
//
// Memory-bound: a row is read once (2 bytes an element) and written once (one
// byte an MXFP8 element, half a byte an MXFP4 one, plus a scale byte per 32);
// the cos/sin table row of a token is shared by its heads and stays in L2.
// A unit is eight consecutive elements (one 16-byte load) of the flat
// rows x (D / 8) unit grid; consecutive lanes take consecutive units, so a
// wave reads 1 KiB of contiguous input per load and the four lanes of a
// 32-element block are lanes 4q .. 4q + 3 of one wave: the block maximum
// takes two lane exchanges.  x is read and the outputs written nontemporally
// (each byte is touched once).
#include "common.hpp"
#include "launch.hpp"

namespace lowbit {

namespace {

// Thread t of the grid takes units t + j * stride, j < UPT (stride = the grid's
// thread count, a multiple of 4, so the four units of a block stay on four
// adjacent lanes): all UPT input loads are issued before any arithmetic.
constexpr int kUnitsPerThread = 4;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

template <int FMT, int LAYOUT>
__global__ __launch_bounds__(256) void rope_quant_kernel(RopeArgs a) {
  constexpr int EMAX = FMT == kMXFP8 ? 8 : 2;      // largest exponent of E4M3 / E2M1
  constexpr int UPT = kUnitsPerThread;
  // unit indices fit 32 bits (the host checks rows x D / 8 < 2^31): one
  // 32-bit division per thread, the later units stepped from the first
  const uint32_t upr = (uint32_t)(a.D / 8);         // 8-element units per row
  const int64_t nblk = a.D / 32;
  const int64_t nope = a.D - a.R;
  const uint32_t units = (uint32_t)(a.rows_grid * upr);
  const uint32_t stride = gridDim.x * 256u;
  const uint32_t u0 = blockIdx.x * 256u + threadIdx.x;
  const uint32_t drow = stride / upr, dk = stride % upr;
  uint32_t r_cur = u0 / upr, k_cur = u0 % upr;

  // every load before any arithmetic (a position and its table row are two
  // dependent round trips; issued for all units together they overlap)
  v4u w[UPT];
  int64_t row_[UPT], k0_[UPT];
  bool live_[UPT], rot_[UPT];
#pragma unroll
  for (int j = 0; j < UPT; j++) {
    const bool in_grid = u0 < units && (uint32_t)j * stride < units - u0;   // u0 + j stride < units
    row_[j] = in_grid ? r_cur : 0;
    k0_[j] = in_grid ? (int64_t)k_cur * 8 : 0;
    live_[j] = in_grid && row_[j] < a.rows;
    rot_[j] = live_[j] && a.R > 0 && k0_[j] + 8 > nope;
    r_cur += drow;                                 // next unit: u + stride
    k_cur += dk;
    if (k_cur >= upr) { k_cur -= upr; r_cur += 1; }
  }
  // loads return in issue order, so the positions (which the table addresses
  // need) go first, then the inputs, then the table entries
  int64_t praw[UPT];
  if (a.R > 0) {
#pragma unroll
    for (int j = 0; j < UPT; j++) {
      const uint32_t t = (uint32_t)row_[j] / (uint32_t)a.heads;
      praw[j] = a.positions[rot_[j] ? t : 0u];
    }
  }
  // branch-free: a unit outside the rows loads row 0 (always present); its
  // values are never stored, and the four lanes of a block share a row, so
  // no value of a live block depends on them.  No branch join or select
  // forces the loads to drain one by one.
#pragma unroll
  for (int j = 0; j < UPT; j++)
    w[j] = __builtin_nontemporal_load(
        reinterpret_cast<const v4u*>(a.x + (live_[j] ? row_[j] * a.D + k0_[j] : 0)));
  // cos / sin of every pair from clamped, always valid table indices (the
  // table is never read outside); pairs outside the rotary slice keep their
  // values (the select follows the arithmetic, so nothing waits on a load
  // before all of them are issued); one uniform branch on R
  float cs[UPT][4], sn[UPT][4];
  if (a.R > 0) {
    int64_t pos[UPT];
#pragma unroll
    for (int j = 0; j < UPT; j++) pos[j] = praw[j] < 0 ? 0 : (praw[j] >= a.P ? a.P - 1 : praw[j]);
    const int64_t half = a.R >> 1;
    // a rotary slice starting on a unit (D - R and R multiples of 8) and a
    // 16-byte aligned table: a unit's four cos and four sin are two vectors
    const bool vec = (nope % 8) == 0 && (a.R % 8) == 0 && (reinterpret_cast<uintptr_t>(a.rope) & 15) == 0;
    if (vec) {
#pragma unroll
      for (int j = 0; j < UPT; j++) {
        int64_t pi = (k0_[j] - nope) >> 1;
        pi = pi < 0 ? 0 : (pi > half - 4 ? half - 4 : pi);
        const float4 c4 = *reinterpret_cast<const float4*>(a.rope + pos[j] * a.R + pi);
        const float4 s4 = *reinterpret_cast<const float4*>(a.rope + pos[j] * a.R + pi + half);
        cs[j][0] = c4.x; cs[j][1] = c4.y; cs[j][2] = c4.z; cs[j][3] = c4.w;
        sn[j][0] = s4.x; sn[j][1] = s4.y; sn[j][2] = s4.z; sn[j][3] = s4.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < UPT; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          int64_t pi = (k0_[j] + 2 * q - nope) >> 1;
          pi = pi < 0 ? 0 : (pi >= half ? half - 1 : pi);
          const float* tab = a.rope + pos[j] * a.R + pi;
          cs[j][q] = tab[0];
          sn[j][q] = tab[half];
        }
    }
  }
#pragma unroll
  for (int j = 0; j < UPT; j++) {
    const int64_t row = row_[j], k0 = k0_[j];
    const bool live = live_[j], in_grid = u0 < units && (uint32_t)j * stride < units - u0;
    float y[8];
    const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      y[2 * q] = bf16_lo(ww[q]);
      y[2 * q + 1] = bf16_hi(ww[q]);
    }
    // inverse rotation of the pairs (k, k + 1) of the last R elements:
    // even' = even c + odd s, odd' = odd c - even s, the second product
    // rounded then one fused multiply-add (pairs outside the slice are left
    // as they are)
    if (a.R > 0) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const bool r = rot_[j] && k0 + 2 * q >= nope;
        const float e = y[2 * q], o = y[2 * q + 1];
        const float e2 = __fmaf_rn(e, cs[j][q], __fmul_rn(o, sn[j][q]));
        const float o2 = __fmaf_rn(o, cs[j][q], -__fmul_rn(e, sn[j][q]));
        y[2 * q] = r ? e2 : e;
        y[2 * q + 1] = r ? o2 : o;
      }
    }
    // block maximum over the four lanes of the block, floored at 1e-10 (the
    // page's max(amax, 1e-10)); the OCP MX scale on it
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; q++) amax = fmaxf(amax, fabsf(y[q]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, 1e-10f);
    float inv;
    const uint32_t sb = mx_block_scale_e<EMAX>(amax, &inv);
#pragma unroll
    for (int q = 0; q < 8; q++) y[q] = __fmul_rn(y[q], inv);   // exact: a power of two
    if (live) {
      if constexpr (FMT == kMXFP8) {
        const uint2 c = e4m3x8(y);
        const v2u cv = {c.x, c.y};
        __builtin_nontemporal_store(cv, reinterpret_cast<v2u*>(a.out_packed + row * a.D + k0));
      } else {
        __builtin_nontemporal_store(e2m1x8(y), reinterpret_cast<uint32_t*>(a.out_packed + row * (a.D / 2) + k0 / 2));
      }
      if ((k0 & 31) == 0) a.out_sf[sf_offset(FMT, LAYOUT, row, k0 / 32, nblk)] = (uint8_t)sb;
    }
    // padded scale layouts: the first unit of each covered row zeroes its
    // padding blocks (every block of a padding row)
    if constexpr (LAYOUT != kLinear) {
      if (in_grid && k0 == 0) {
        const int64_t nblk_pad = sf_pad_blocks(LAYOUT, nblk);
        for (int64_t kb = (row < a.rows ? nblk : 0); kb < nblk_pad; kb++)
          a.out_sf[sf_offset(FMT, LAYOUT, row, kb, nblk)] = 0;
      }
    }
  }
}

template <int FMT, int LAYOUT>
hipError_t launch(const RopeArgs& a, hipStream_t s) {
  const int64_t units = a.rows_grid * (a.D / 8);
  const unsigned grid = (unsigned)((units + 256 * kUnitsPerThread - 1) / (256 * kUnitsPerThread));
  hipLaunchKernelGGL((rope_quant_kernel<FMT, LAYOUT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_quant(const RopeArgs& args, int fmt, int layout, hipStream_t s) {
  RopeArgs a = args;
  a.rows_grid = sf_pad_rows(layout, a.rows);
  if (a.rows_grid == 0) return hipSuccess;
  if (fmt == kMXFP8) return launch<kMXFP8, kLinear>(a, s);
  if (layout == kTiled) return launch<kMXFP4, kTiled>(a, s);
  if (layout == kSwz128) return launch<kMXFP4, kSwz128>(a, s);
  return launch<kMXFP4, kLinear>(a, s);
}

}  // namespace lowbit
