// quant.hip -- the memory-bound row kernels of liblowbit (gfx950):
//   * fused add + RMSNorm + FP4 quantization (FlashInfer page,
//     cute_dsl/add_rmsnorm_fp4quant.py, AddRMSNormFP4QuantKernel phases 1-3);
//   * plain FP4 quantization of a bf16 tensor and its dequantization (FlashRT
//     fp4-gemm README, quantize_fp4_sfa_* / dequantize_fp4_sfa_*);
//   * the same three for MXFP8 (E4M3 elements, one byte each, UE8M0 32-blocks;
//     the vLLM page's FusedWoAKernel quantizes to this format).
//
// Two forms.  Many rows (M >= 256) of up to 16384 elements take one
// workgroup per row (row_wg_kernel, below).  Otherwise a row is owned by WPR
// wavefronts (1, 2 or 4) of a 256-thread workgroup; inside a wave, lane l owns
// quantization blocks l, l+64, ... (NBL of them) of the wave's stretch of the
// row.  In both, the whole row stays in registers as bf16 between the
// reduction and the quantization, so HBM sees exactly: x and r read once, r
// written once, the packed codes and the scales written once.  The sum of squares is kept in
// fp64 per lane (each fp32 h^2 is exact there), reduced across the wave with
// shuffles and across the row's waves through LDS.
//
// Floating-point order follows the page's kernel exactly, without
// contraction: h = fl32(x + r), rstd = fl32(1 / sqrt(S / H + eps)) from the
// fp64 S, y = fl32(fl32(bf16(h) * rstd) * w), then the block scale rule.
#include "common.hpp"
#include "launch.hpp"

namespace lowbit {

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte vectors per quantization block of bf16 values
template <int B> struct BlockVec { static constexpr int kVecs = B * 2 / 16; };

struct RowArgs {
  const uint16_t* x;       // fused: input; quantize: the tensor
  uint16_t* residual;      // fused only
  const uint16_t* w;       // fused only
  int64_t M, H;
  int64_t rows_grid;       // rows covered by the grid (>= M; TILED pads to 32)
  float eps;
  int layout;
  const float* gs;         // NVFP4 global scale or nullptr
  uint8_t* out_packed;
  uint8_t* out_sf;
  uint8_t* out_sf_lin;     // nullptr, or a LINEAR copy of the scales beside TILED out_sf
};

// Quantize the NBL blocks a lane owns (values y in registers) and store them.
template <int FMT>
__device__ __forceinline__ void quant_store_block(const float* y, float gs, int64_t row, int64_t kb,
                                                  int64_t nblk, const RowArgs& a) {
  constexpr int B = FmtTraits<FMT>::B;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < B; i++) amax = fmaxf(amax, fabsf(y[i]));
  float inv;
  uint32_t sb = e4m3_scaled(FMT) ? nv_block_scale(amax, gs, &inv)
                : (FMT == kMXFP8) ? mx_block_scale_e<8>(amax, &inv) : mx_block_scale(amax, &inv);
  float v[B];
#pragma unroll
  for (int i = 0; i < B; i++) v[i] = __fmul_rn(y[i], inv);
  if constexpr (FMT == kMXFP8) {
    // one E4M3 byte per element: the block's 32 bytes as two 16-byte stores
    uint8_t* dst = a.out_packed + row * a.H + kb * B;
    const uint2 c0 = e4m3x8(v), c1 = e4m3x8(v + 8), c2 = e4m3x8(v + 16), c3 = e4m3x8(v + 24);
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(c0.x, c0.y, c1.x, c1.y);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(c2.x, c2.y, c3.x, c3.y);
    a.out_sf[sf_offset(FMT, a.layout, row, kb, nblk)] = (uint8_t)sb;
    if (a.out_sf_lin != nullptr) a.out_sf_lin[row * nblk + kb] = (uint8_t)sb;
    return;
  }
  uint8_t* dst = a.out_packed + row * (a.H / 2) + kb * (B / 2);
  if constexpr (B == 16) {
    uint2 p;
    p.x = e2m1x8(v);
    p.y = e2m1x8(v + 8);
    *reinterpret_cast<uint2*>(dst) = p;
  } else {
    uint4 p;
    p.x = e2m1x8(v);
    p.y = e2m1x8(v + 8);
    p.z = e2m1x8(v + 16);
    p.w = e2m1x8(v + 24);
    *reinterpret_cast<uint4*>(dst) = p;
  }
  a.out_sf[sf_offset(FMT, a.layout, row, kb, nblk)] = (uint8_t)sb;
  if (a.out_sf_lin != nullptr) a.out_sf_lin[row * nblk + kb] = (uint8_t)sb;
}

// FUSED: add + RMSNorm + quant.  Otherwise: quantize x as it is.  F16: the
// 16-bit tensors (x, residual, weight) are fp16, else bf16.
template <int FMT, int NBL, int WPR, bool FUSED, bool F16>
__global__ __launch_bounds__(kThreads) void row_quant_kernel(RowArgs a) {
  constexpr int B = FmtTraits<FMT>::B;
  constexpr int VECS = BlockVec<B>::kVecs;
  constexpr int ROWS_PER_WG = (kThreads / kWave) / WPR;
  __shared__ double red[kThreads / kWave];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int wave_in_row = wave % WPR;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_WG + wave / WPR;
  const int64_t nblk = a.H / B;
  // this wave's stretch of blocks
  const int64_t per_wave = (nblk + WPR - 1) / WPR;
  const int64_t kb0 = wave_in_row * per_wave;
  const int64_t kb_end = (kb0 + per_wave < nblk) ? kb0 + per_wave : nblk;
  const bool live = row < a.M;

  // h (or x) of the lane's blocks in the input format, two values per word
  uint32_t hb[NBL][B / 2];
  double ss = 0.0;

  if (live) {
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int64_t kb = kb0 + lane + (int64_t)i * kWave;
      if (kb < kb_end) {
        const u32x4* px = reinterpret_cast<const u32x4*>(a.x + row * a.H + kb * B);
        u32x4 xv[VECS];
#pragma unroll
        for (int v = 0; v < VECS; v++) xv[v] = __builtin_nontemporal_load(px + v);
        if constexpr (FUSED) {
          u32x4* pr = reinterpret_cast<u32x4*>(a.residual + row * a.H + kb * B);
          u32x4 rv[VECS];
#pragma unroll
          for (int v = 0; v < VECS; v++) rv[v] = __builtin_nontemporal_load(pr + v);
#pragma unroll
          for (int v = 0; v < VECS; v++) {
            const uint32_t* xw = reinterpret_cast<const uint32_t*>(&xv[v]);
            const uint32_t* rw = reinterpret_cast<const uint32_t*>(&rv[v]);
#pragma unroll
            for (int j = 0; j < 4; j++) {
              float h0 = __fadd_rn(in_lo<F16>(xw[j]), in_lo<F16>(rw[j]));
              float h1 = __fadd_rn(in_hi<F16>(xw[j]), in_hi<F16>(rw[j]));
              ss = __fma_rn((double)h0, (double)h0, ss);
              ss = __fma_rn((double)h1, (double)h1, ss);
              hb[i][v * 4 + j] = pack_in2<F16>(h0, h1);
            }
          }
          // residual <- bf16(h), same positions
#pragma unroll
          for (int v = 0; v < VECS; v++) {
            u32x4 o = {hb[i][v * 4 + 0], hb[i][v * 4 + 1], hb[i][v * 4 + 2], hb[i][v * 4 + 3]};
            __builtin_nontemporal_store(o, pr + v);
          }
        } else {
#pragma unroll
          for (int v = 0; v < VECS; v++) {
            hb[i][v * 4 + 0] = xv[v].x;
            hb[i][v * 4 + 1] = xv[v].y;
            hb[i][v * 4 + 2] = xv[v].z;
            hb[i][v * 4 + 3] = xv[v].w;
          }
        }
      }
    }
  }

  float rstd = 1.0f;
  if constexpr (FUSED) {
    ss = wave_sum_f64(ss);
    if constexpr (WPR > 1) {
      if (lane == 0) red[wave] = ss;
      __syncthreads();
      const int first = (wave / WPR) * WPR;
      ss = 0.0;
#pragma unroll
      for (int w = 0; w < WPR; w++) ss += red[first + w];
    }
    rstd = (float)(1.0 / sqrt(ss / (double)a.H + (double)a.eps));
  }

  const float gs = (e4m3_scaled(FMT) && a.gs != nullptr) ? *a.gs : 1.0f;

  if (live) {
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int64_t kb = kb0 + lane + (int64_t)i * kWave;
      if (kb < kb_end) {
        float y[B];
        if constexpr (FUSED) {
          const uint4* pw = reinterpret_cast<const uint4*>(a.w + kb * B);
#pragma unroll
          for (int v = 0; v < VECS; v++) {
            uint4 wv = pw[v];
            const uint32_t* ww = reinterpret_cast<const uint32_t*>(&wv);
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const uint32_t h2 = hb[i][v * 4 + j];
              y[v * 8 + 2 * j] = __fmul_rn(__fmul_rn(in_lo<F16>(h2), rstd), in_lo<F16>(ww[j]));
              y[v * 8 + 2 * j + 1] = __fmul_rn(__fmul_rn(in_hi<F16>(h2), rstd), in_hi<F16>(ww[j]));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < B / 2; j++) {
            y[2 * j] = in_lo<F16>(hb[i][j]);
            y[2 * j + 1] = in_hi<F16>(hb[i][j]);
          }
        }
        quant_store_block<FMT>(y, gs, row, kb, nblk, a);
      }
    }
  }

  // TILED / SWZ128 padding: zero the scale bytes of blocks nblk..nblk_pad-1
  // of every covered row, and all bytes of the rows M..rows_grid-1.
  if (a.layout != kLinear && row < a.rows_grid) {
    const int64_t nblk_pad = sf_pad_blocks(a.layout, nblk);
    if (live) {
      const int64_t pad = nblk_pad - nblk;
      if (wave_in_row == 0 && lane < pad) a.out_sf[sf_offset(FMT, a.layout, row, nblk + lane, nblk)] = 0;
    } else {
      for (int64_t kb = kb0 + lane; kb < ((wave_in_row == WPR - 1) ? nblk_pad : kb_end); kb += kWave)
        a.out_sf[sf_offset(FMT, a.layout, row, kb, nblk)] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// Row-per-workgroup form for many rows of at most 16384 elements.  A row is
// H/8 vectors of 8 bf16 (16 B); the workgroup has T = 64 * NW threads and
// thread t owns vectors t + jT, j < V, so that every load and store
// instruction of a wave covers one contiguous 1 KiB span (256 B of codes) and
// each thread keeps 2V 16-byte loads of x and r in flight.  V = 2, NW =
// ceil(H / 1024); for 4096 < H <= 6144 over more than 1280 rows, V = 3 and
// NW = 4 instead of 5 or 6.
// Resident workgroups (up to eight 4-wave ones per CU) are what keeps enough
// bytes in flight to stream HBM: measured 20.5 us on 4096 x 4096 NVFP4 against
// 25.3 us for a form with persistent waves carrying several rows, and 18 us for
// a plain stream of the same x and r reads and residual writes without the
// codes.  The row's sum of squares is reduced with a wave butterfly and
// across the NW waves through LDS, in wave order.  A quantization block is B/8
// adjacent lanes (2 for NVFP4, 4 for MXFP4): its amax is exchanged with one or
// two lane shuffles and its first lane writes the scale byte.  Workgroups of
// the TILED padding rows (M .. rows_grid - 1) only zero their scale bytes.
// ---------------------------------------------------------------------------
constexpr int kWgMinRows = 256;     // fewer rows: the row-split form has more parallelism
constexpr int kWgMaxWaves = 16;     // H <= 16384
constexpr int kWgVecs = 2;          // 16-byte vectors per thread and tensor (3 for 4096 < H <= 6144)

// TILED: the row of workgroup b.  Workgroups start on XCD b % 8; this order
// puts the 32 rows of each 32-row scale group on one XCD, whose L2 then
// merges the group's scale bytes into whole lines before writing them back
// (in launch order, each line was written back partially by up to 8 L2s).
// A bijection on [0, G): blocks past the last multiple of 256 keep their row.
__device__ __forceinline__ int64_t tiled_row_of_block(int64_t b, int64_t G) {
  const int64_t full = G & ~int64_t(255);
  if (b >= full) return b;
  const int64_t x = b & 7, i = b >> 3;
  return ((x + 8 * (i >> 5)) << 5) + (i & 31);
}

template <int FMT, int NW, int V, bool FUSED, bool F16>
__global__ __launch_bounds__(NW * kWave) void row_wg_kernel(RowArgs a) {
  constexpr int B = FmtTraits<FMT>::B;
  constexpr int LPB = B / 8;   // lanes per block
  constexpr int T = NW * kWave;
  __shared__ double part[NW];
  const int t = threadIdx.x, lane = t % kWave;
  const int64_t row = (a.layout == kTiled) ? tiled_row_of_block(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t H = a.H, nblk = H / B, nvec = H / 8;
  const int64_t nblk_pad = sf_pad_blocks(a.layout, nblk);
  if (row >= a.M) {
    // TILED / SWZ128 padding row: every scale byte zero
    for (int64_t kb = t; kb < nblk_pad; kb += T) a.out_sf[sf_offset(FMT, a.layout, row, kb, nblk)] = 0;
    return;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const u32x4* xr = reinterpret_cast<const u32x4*>(a.x + row * H);
  u32x4* rr = reinterpret_cast<u32x4*>(a.residual + row * H);
  u32x4 xv[V], rv[V], wv[V];
#pragma unroll
  for (int j = 0; j < V; j++) {
    const int q = j * T + t;
    xv[j] = zero;
    rv[j] = zero;
    wv[j] = zero;
    if (q < nvec) {
      // nontemporal: x and r are read once (measured faster than cached loads
      // when the inputs are not in the last-level cache)
      xv[j] = __builtin_nontemporal_load(xr + q);
      if constexpr (FUSED) {
        rv[j] = __builtin_nontemporal_load(rr + q);
        wv[j] = reinterpret_cast<const u32x4*>(a.w)[q];   // shared by every row: cached
      }
    }
  }
  const float gs = (e4m3_scaled(FMT) && a.gs != nullptr) ? *a.gs : 1.0f;
  float rstd = 1.0f;
  if constexpr (FUSED) {
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < V; j++) {
      u32x4 hw;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const float h0 = __fadd_rn(in_lo<F16>(xv[j][k]), in_lo<F16>(rv[j][k]));
        const float h1 = __fadd_rn(in_hi<F16>(xv[j][k]), in_hi<F16>(rv[j][k]));
        ss = __fma_rn((double)h0, (double)h0, ss);
        ss = __fma_rn((double)h1, (double)h1, ss);
        hw[k] = pack_in2<F16>(h0, h1);
      }
      xv[j] = hw;   // the row's h in the input format, kept for the second pass
      if (j * T + t < nvec) __builtin_nontemporal_store(hw, rr + j * T + t);
    }
    ss = wave_sum_f64(ss);
    if constexpr (NW > 1) {
      if (lane == 0) part[t / kWave] = ss;
      __syncthreads();
      ss = part[0];
#pragma unroll
      for (int i = 1; i < NW; i++) ss += part[i];
    }
    rstd = (float)(1.0 / sqrt(ss / (double)H + (double)a.eps));
  }
  uint32_t* const code_row = reinterpret_cast<uint32_t*>(a.out_packed + row * (H / 2));
  uint8_t* const sf_row = (a.layout == kLinear)
                              ? a.out_sf + row * nblk
                              : a.out_sf + (((row >> 5) * (nblk_pad >> 3)) << 8) + ((row & 31) << 2);
#pragma unroll
  for (int j = 0; j < V; j++) {
    const int q = j * T + t;
    float y[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      if constexpr (FUSED) {
        y[2 * k] = __fmul_rn(__fmul_rn(in_lo<F16>(xv[j][k]), rstd), in_lo<F16>(wv[j][k]));
        y[2 * k + 1] = __fmul_rn(__fmul_rn(in_hi<F16>(xv[j][k]), rstd), in_hi<F16>(wv[j][k]));
      } else {
        y[2 * k] = in_lo<F16>(xv[j][k]);
        y[2 * k + 1] = in_hi<F16>(xv[j][k]);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(y[i]));
    // the block's lanes are all inside the row or all past it (H % B == 0, T % 64 == 0)
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    if constexpr (LPB == 4) amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    float inv;
    const uint32_t sb = e4m3_scaled(FMT) ? nv_block_scale(amax, gs, &inv)
                        : (FMT == kMXFP8) ? mx_block_scale_e<8>(amax, &inv) : mx_block_scale(amax, &inv);
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] = __fmul_rn(y[i], inv);
    if (q < nvec) {
      if constexpr (FMT == kMXFP8)   // one E4M3 byte per element: 8 bytes per vector
        reinterpret_cast<uint2*>(a.out_packed + row * H)[q] = e4m3x8(y);
      else
        code_row[q] = e2m1x8(y);
      if (q % LPB == 0) {
        const int kb = q / LPB, jj = kb & 7;
        const int in_grp = (FMT == kNVFP4) ? ((jj >> 2) << 7) + (jj & 3)
                                           : (((jj >> 1) & 1) << 7) + (jj & 1) + ((jj >> 2) << 1);
        if (a.layout == kSwz128)
          a.out_sf[sf_offset(FMT, kSwz128, row, kb, nblk)] = (uint8_t)sb;
        else
          sf_row[(a.layout == kLinear) ? kb : ((kb >> 3) << 8) + in_grp] = (uint8_t)sb;
        if (a.out_sf_lin != nullptr) a.out_sf_lin[row * nblk + kb] = (uint8_t)sb;
      }
    }
  }
  // TILED / SWZ128: the row's padding blocks nblk .. nblk_pad - 1 are zero
  if (a.layout != kLinear && t < nblk_pad - nblk) a.out_sf[sf_offset(FMT, a.layout, row, nblk + t, nblk)] = 0;
}

template <int FMT, int NW, bool FUSED, bool F16, int V = kWgVecs>
hipError_t launch_wg(const RowArgs& a, hipStream_t s) {
  if (a.rows_grid == 0) return hipSuccess;
  hipLaunchKernelGGL((row_wg_kernel<FMT, NW, V, FUSED, F16>), dim3((unsigned)a.rows_grid), dim3(NW * kWave), 0, s,
                     a);
  return hipGetLastError();
}

template <int FMT, int NBL, int WPR, bool FUSED, bool F16>
hipError_t launch_row(const RowArgs& a, hipStream_t s) {
  constexpr int ROWS_PER_WG = (kThreads / kWave) / WPR;
  int64_t grid = (a.rows_grid + ROWS_PER_WG - 1) / ROWS_PER_WG;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((row_quant_kernel<FMT, NBL, WPR, FUSED, F16>), dim3((unsigned)grid), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

// Many rows of at most 16384 elements: a workgroup per row.  Otherwise pick
// (WPR, NBL) of the row-split form for a row of nblk blocks: one wave per row
// when there are many rows, a row spread over up to 4 waves when there are few.
template <int FMT, bool FUSED, bool F16>
hipError_t dispatch_row(const RowArgs& a, hipStream_t s) {
  constexpr int MAXNBL = (FMT == kNVFP4) ? 8 : 4;   // MXFP4, MXFP8: 32-blocks
  const int64_t nblk = a.H / FmtTraits<FMT>::B;
  const int64_t nw = (a.H + kWgVecs * 8 * kWave - 1) / (kWgVecs * 8 * kWave);
  if (a.M >= kWgMinRows && nw <= kWgMaxWaves && a.rows_grid <= 0x7FFFFFFF) {
    // 4096 < H <= 6144: three vectors per thread make the workgroup 4 waves
    // wide instead of 5 or 6, so eight of them (32 waves) stay resident per
    // CU.  Only for more rows than the wider workgroups keep resident in one
    // pass (five per CU): with fewer, the narrower form only loses threads
    // (measured 2048 x 5120: 16.1 -> 15.3 us, 2048 x 6144: 19.2 -> 17.7 us;
    // 300 x 5632: 13.5 -> 14.0 us).  Rows of 4096 keep V = 2 in 4 waves: all
    // 4096 rows of 4096 x 4096 resident at once, as 2 waves with V = 4 or one
    // with V = 8, measured 23.2 and 28.6 us against 21.1 us.
    if ((nw == 5 || nw == 6) && a.rows_grid > 5 * 256) return launch_wg<FMT, 4, FUSED, F16, 3>(a, s);
    switch (nw) {
      case 1: return launch_wg<FMT, 1, FUSED, F16>(a, s);
      case 2: return launch_wg<FMT, 2, FUSED, F16>(a, s);
      case 3: return launch_wg<FMT, 3, FUSED, F16>(a, s);
      case 4: return launch_wg<FMT, 4, FUSED, F16>(a, s);
      case 5: return launch_wg<FMT, 5, FUSED, F16>(a, s);
      case 6: return launch_wg<FMT, 6, FUSED, F16>(a, s);
      case 7: return launch_wg<FMT, 7, FUSED, F16>(a, s);
      case 8: return launch_wg<FMT, 8, FUSED, F16>(a, s);
      case 9: return launch_wg<FMT, 9, FUSED, F16>(a, s);
      case 10: return launch_wg<FMT, 10, FUSED, F16>(a, s);
      case 11: return launch_wg<FMT, 11, FUSED, F16>(a, s);
      case 12: return launch_wg<FMT, 12, FUSED, F16>(a, s);
      case 13: return launch_wg<FMT, 13, FUSED, F16>(a, s);
      case 14: return launch_wg<FMT, 14, FUSED, F16>(a, s);
      case 15: return launch_wg<FMT, 15, FUSED, F16>(a, s);
      default: return launch_wg<FMT, 16, FUSED, F16>(a, s);
    }
  }
  int wpr = (a.M >= 1024) ? 1 : 4;
  if (nblk <= 64) wpr = 1;
  while (wpr < 4 && (nblk + 64 * wpr - 1) / (64 * wpr) > MAXNBL) wpr *= 2;
  int64_t nbl = (nblk + 64 * wpr - 1) / (64 * wpr);
  if (nbl > MAXNBL) return hipErrorInvalidValue;
#define LB_CASE(W, N)                                                            \
  if (wpr == W && nbl == N) return launch_row<FMT, N, W, FUSED, F16>(a, s);
#define LB_ALL(W) LB_CASE(W, 1) LB_CASE(W, 2) LB_CASE(W, 3) LB_CASE(W, 4)
  LB_ALL(1) LB_ALL(2) LB_ALL(4)
  if constexpr (MAXNBL == 8) {
#define LB_HI(W) LB_CASE(W, 5) LB_CASE(W, 6) LB_CASE(W, 7) LB_CASE(W, 8)
    LB_HI(1) LB_HI(2) LB_HI(4)
#undef LB_HI
  }
#undef LB_ALL
#undef LB_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Dequantize: one lane per block; bf16 output, or fp16 with F16 (both
// nearest-even from the binary32 value; fp16 overflows to infinity).
// ---------------------------------------------------------------------------
template <int FMT, bool F16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* packed, const uint8_t* sf,
                                                           int64_t rows, int64_t K, int layout,
                                                           const float* gsp, uint16_t* out) {
  constexpr int B = FmtTraits<FMT>::B;
  const int64_t nblk = K / B;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= rows * nblk) return;
  const int64_t row = t / nblk, kb = t % nblk;
  const uint32_t sb = sf[sf_offset(FMT, layout, row, kb, nblk)];
  const float scale = e4m3_scaled(FMT) ? e4m3_to_f32(sb) : ue8m0_to_f32(sb);
  const float gs = (e4m3_scaled(FMT) && gsp != nullptr) ? *gsp : 1.0f;
  uint16_t* dst = out + row * K + kb * B;
  if constexpr (FMT == kMXFP8) {
    // 32 E4M3 bytes; value * 2^e is exact in fp32 and has 4 significant bits
    const uint4* src8 = reinterpret_cast<const uint4*>(packed + row * K + kb * B);
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint4 p = src8[h];
      const uint32_t w4[4] = {p.x, p.y, p.z, p.w};
      uint32_t o[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint32_t wd = w4[j >> 1], sh = 16 * (j & 1);
        o[j] = pack_in2<F16>(__fmul_rn(e4m3_to_f32((wd >> sh) & 0xFF), scale),
                             __fmul_rn(e4m3_to_f32((wd >> (sh + 8)) & 0xFF), scale));
      }
      uint4* d4 = reinterpret_cast<uint4*>(dst + h * 16);
      d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
      d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    return;
  }
  const uint8_t* src = packed + row * (K / 2) + kb * (B / 2);
#pragma unroll
  for (int q = 0; q < B / 16; q++) {
    uint2 p = *reinterpret_cast<const uint2*>(src + q * 8);
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      uint32_t byte = ((j < 4 ? p.x : p.y) >> (8 * (j & 3))) & 0xFF;
      float v0 = __fmul_rn(e2m1_to_f32(byte & 15), scale);   // exact
      float v1 = __fmul_rn(e2m1_to_f32(byte >> 4), scale);
      if (e4m3_scaled(FMT)) { v0 = __fdiv_rn(v0, gs); v1 = __fdiv_rn(v1, gs); }
      o[j] = pack_in2<F16>(v0, v1);
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst + q * 16);
    d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

}  // namespace

hipError_t launch_add_rmsnorm_quant(const uint16_t* x, uint16_t* residual, const uint16_t* w, int64_t M,
                                    int64_t H, float eps, int fmt, int layout, const float* gs,
                                    uint8_t* out_packed, uint8_t* out_sf, uint8_t* out_sf_lin, int in_f16,
                                    hipStream_t s) {
  RowArgs a{x, residual, w, M, H, M, eps, layout, gs, out_packed, out_sf, out_sf_lin};
  a.rows_grid = sf_pad_rows(layout, M);
  if (fmt == kMXFP8) return in_f16 ? dispatch_row<kMXFP8, true, true>(a, s) : dispatch_row<kMXFP8, true, false>(a, s);
  if (fmt == kNV32) return in_f16 ? dispatch_row<kNV32, true, true>(a, s) : dispatch_row<kNV32, true, false>(a, s);
  if (in_f16) return fmt == kNVFP4 ? dispatch_row<kNVFP4, true, true>(a, s) : dispatch_row<kMXFP4, true, true>(a, s);
  return fmt == kNVFP4 ? dispatch_row<kNVFP4, true, false>(a, s) : dispatch_row<kMXFP4, true, false>(a, s);
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t K, int fmt, int layout,
                           const float* gs, uint8_t* out_packed, uint8_t* out_sf, int in_f16, hipStream_t s) {
  RowArgs a{x, nullptr, nullptr, rows, K, rows, 0.0f, layout, gs, out_packed, out_sf, nullptr};
  a.rows_grid = sf_pad_rows(layout, rows);
  if (fmt == kMXFP8) return in_f16 ? dispatch_row<kMXFP8, false, true>(a, s) : dispatch_row<kMXFP8, false, false>(a, s);
  if (fmt == kNV32) return in_f16 ? dispatch_row<kNV32, false, true>(a, s) : dispatch_row<kNV32, false, false>(a, s);
  if (in_f16) return fmt == kNVFP4 ? dispatch_row<kNVFP4, false, true>(a, s) : dispatch_row<kMXFP4, false, true>(a, s);
  return fmt == kNVFP4 ? dispatch_row<kNVFP4, false, false>(a, s) : dispatch_row<kMXFP4, false, false>(a, s);
}

template <bool F16>
static void dequant_fmt(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K, int fmt, int layout,
                        const float* gs, uint16_t* out, unsigned grid, hipStream_t s) {
  if (fmt == kNVFP4)
    hipLaunchKernelGGL((dequant_kernel<kNVFP4, F16>), dim3(grid), dim3(kThreads), 0, s, packed, sf, rows, K,
                       layout, gs, out);
  else if (fmt == kNV32)
    hipLaunchKernelGGL((dequant_kernel<kNV32, F16>), dim3(grid), dim3(kThreads), 0, s, packed, sf, rows, K,
                       layout, gs, out);
  else if (fmt == kMXFP8)
    hipLaunchKernelGGL((dequant_kernel<kMXFP8, F16>), dim3(grid), dim3(kThreads), 0, s, packed, sf, rows, K,
                       layout, gs, out);
  else
    hipLaunchKernelGGL((dequant_kernel<kMXFP4, F16>), dim3(grid), dim3(kThreads), 0, s, packed, sf, rows, K,
                       layout, gs, out);
}

hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K, int fmt,
                             int layout, const float* gs, uint16_t* out, int out_f16, hipStream_t s) {
  const int64_t nblk = K / (fmt == kNVFP4 ? 16 : 32);
  const int64_t n = rows * nblk;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
  if (out_f16) dequant_fmt<true>(packed, sf, rows, K, fmt, layout, gs, out, grid, s);
  else dequant_fmt<false>(packed, sf, rows, K, fmt, layout, gs, out, grid, s);
  return hipGetLastError();
}

}  // namespace lowbit
