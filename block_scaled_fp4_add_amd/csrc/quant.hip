// quant.hip -- the memory-bound row kernels of liblowbit (gfx950):
//   * fused add + RMSNorm + FP4 quantization (FlashInfer page,
//     cute_dsl/add_rmsnorm_fp4quant.py, AddRMSNormFP4QuantKernel phases 1-3);
//   * plain FP4 quantization of a bf16 tensor and its dequantization (FlashRT
//     fp4-gemm README, quantize_fp4_sfa_* / dequantize_fp4_sfa_*).
//
// Two forms.  Many rows (M >= 256) of up to 6144 elements take the pipelined
// form (row_pipe_kernel, below).  Otherwise a row is owned by WPR wavefronts
// (1, 2 or 4) of a 256-thread workgroup; inside a wave, lane l owns
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
  uint32_t sb = (FMT == kNVFP4) ? nv_block_scale(amax, gs, &inv) : mx_block_scale(amax, &inv);
  float v[B];
#pragma unroll
  for (int i = 0; i < B; i++) v[i] = __fmul_rn(y[i], inv);
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
}

// FUSED: add + RMSNorm + quant.  Otherwise: quantize x as it is.
template <int FMT, int NBL, int WPR, bool FUSED>
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

  // bf16 h (or x) of the lane's blocks, two values per word
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
              float h0 = __fadd_rn(bf16_lo(xw[j]), bf16_lo(rw[j]));
              float h1 = __fadd_rn(bf16_hi(xw[j]), bf16_hi(rw[j]));
              ss = __fma_rn((double)h0, (double)h0, ss);
              ss = __fma_rn((double)h1, (double)h1, ss);
              hb[i][v * 4 + j] = pack_bf16x2(h0, h1);
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

  const float gs = (FMT == kNVFP4 && a.gs != nullptr) ? *a.gs : 1.0f;

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
              y[v * 8 + 2 * j] = __fmul_rn(__fmul_rn(bf16_lo(h2), rstd), bf16_lo(ww[j]));
              y[v * 8 + 2 * j + 1] = __fmul_rn(__fmul_rn(bf16_hi(h2), rstd), bf16_hi(ww[j]));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < B / 2; j++) {
            y[2 * j] = bf16_lo(hb[i][j]);
            y[2 * j + 1] = bf16_hi(hb[i][j]);
          }
        }
        quant_store_block<FMT>(y, gs, row, kb, nblk, a);
      }
    }
  }

  // TILED padding: zero the scale bytes of blocks nblk..8*ceil(nblk/8)-1 of
  // every covered row, and all bytes of the rows M..rows_grid-1.
  if (a.layout == kTiled && row < a.rows_grid) {
    const int64_t nblk_pad = ((nblk + 7) >> 3) << 3;
    if (live) {
      const int64_t pad = nblk_pad - nblk;
      if (wave_in_row == 0 && lane < pad) a.out_sf[sf_offset(FMT, kTiled, row, nblk + lane, nblk)] = 0;
    } else {
      for (int64_t kb = kb0 + lane; kb < ((wave_in_row == WPR - 1) ? nblk_pad : kb_end); kb += kWave)
        a.out_sf[sf_offset(FMT, kTiled, row, kb, nblk)] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined form for many rows of at most 12 * 512 elements.  Waves are
// persistent over rows (row = wave id, + waves, ...) and stream each row in
// chunks of 512 elements with PIPE chunks of x and r in flight: the residual
// of a chunk is written as soon as its loads land, and the last chunks of a
// row already fetch the first chunks of the wave's next row, so that HBM sees
// a steady mix of reads and writes instead of a read phase and a write phase.
// The row's bf16 h stays in registers (4 VGPRs per chunk) for the second
// pass, which quantizes and stores the codes once the row's sum of squares
// is known.  In chunk v lane l holds the 8 elements at v*512 + 8l, so every
// load and store instruction covers one contiguous span (16 B per lane of
// bf16, 4 B per lane of codes).  A block is B/8 adjacent lanes (2 for NVFP4,
// 4 for MXFP4): its amax is exchanged with one or two lane shuffles and its
// first lane writes the scale byte.  The RMSNorm weight row is staged once
// per workgroup in LDS.
// ---------------------------------------------------------------------------
constexpr int kPipeChunk = 512;          // elements per wave-wide chunk
constexpr int kPipeMaxChunks = 12;       // H <= 6144
constexpr int kPipeMinRows = 256;        // fewer rows: the row-split form has more parallelism
// Measured on the 4096 x 4096 and 2048 x 5120 NVFP4 producers: two waves
// per SIMD (registers for the row's bf16 h, 4 per chunk, and the loads in
// flight) with three to four chunks in flight beat deeper prefetch and more
// waves.  The depth divides the row's chunk count: chunk c of every row then
// lives in buffer slot c % depth, also when the last chunks of a row fetch
// the first chunks of the next.
constexpr int pipe_depth(int ch) {
  return ch % 4 == 0 ? 4 : ch % 3 == 0 ? 3 : ch == 10 ? 5 : ch % 2 == 0 ? 2 : ch <= 7 ? ch : 1;
}
constexpr int kPipeWgsPerCu = 2;     // 4-wave workgroups per CU = waves per SIMD
constexpr int kCUs = 256;

template <int FMT, int CH, bool FUSED>
__global__ __launch_bounds__(kThreads, kPipeWgsPerCu) void row_pipe_kernel(RowArgs a) {
  constexpr int B = FmtTraits<FMT>::B;
  constexpr int LPB = B / 8;   // lanes per block
  constexpr int P = pipe_depth(CH);
  static_assert(CH % P == 0, "the depth must divide the chunk count");
  __shared__ u32x4 wl[FUSED ? CH * kPipeChunk / 8 : 1];
  const int lane = threadIdx.x % kWave;
  // wave-uniform row indices: row base addresses stay scalar, one per-lane offset serves every chunk
  const int64_t wid = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave));
  const int64_t nw = (int64_t)gridDim.x * (kThreads / kWave);
  const int64_t H = a.H, nblk = H / B;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // chunk v of `row` into buffer slot (zeros past the row's end or past M)
  u32x4 bx[P], br[P];
  // only the last chunk of a row can be partial (lanes past H are idle)
  auto in_row = [&](int v, int ln) { return v < CH - 1 || v * kPipeChunk + ln * 8 < H; };
  auto fetch = [&](int64_t row, int v, int slot, int ln) {
    bx[slot] = zero;
    if constexpr (FUSED) br[slot] = zero;
    if (row < a.M && in_row(v, ln)) {
      // nontemporal: x and r are read once (measured faster than cached loads
      // when the inputs are not in the last-level cache)
      bx[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x + row * H) + v * (kPipeChunk / 8) + ln);
      if constexpr (FUSED)
        br[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.residual + row * H) + v * (kPipeChunk / 8) + ln);
    }
  };

  int64_t row = wid;
#pragma unroll
  for (int p = 0; p < P; p++) fetch(row, p, p, lane);
  // the weight row goes to LDS while the first chunks are in flight
  if constexpr (FUSED) {
    for (int64_t i = threadIdx.x; i < H / 8; i += kThreads) wl[i] = reinterpret_cast<const u32x4*>(a.w)[i];
    __syncthreads();
  }
  const float gs = (FMT == kNVFP4 && a.gs != nullptr) ? *a.gs : 1.0f;
  for (; row < a.M; row += nw) {
    // the lane index, re-defined opaquely per row: per-chunk lane offsets are
    // recomputed in the loop instead of being hoisted and held for all chunks
    int ln = lane;
    asm volatile("" : "+v"(ln));
    u32x4 hb[CH];
    double ss = 0.0;
    u32x4* const res_row = reinterpret_cast<u32x4*>(a.residual + row * H);
    uint32_t* const code_row = reinterpret_cast<uint32_t*>(a.out_packed + row * (H / 2));
    // the row's scale bytes: a scalar base and a 32-bit per-block offset
    uint8_t* const sf_row = (a.layout == kLinear)
                                ? a.out_sf + row * nblk
                                : a.out_sf + (((row >> 5) * ((nblk + 7) >> 3)) << 8) + ((row & 31) << 2);
#pragma unroll
    for (int v = 0; v < CH; v++) {
      const u32x4 xv = bx[v % P], rv = br[v % P];
      // refill the slot: chunk v + P of this row, or the next row's first chunks
      if (v + P < CH) fetch(row, v + P, v % P, ln); else fetch(row + nw, v + P - CH, v % P, ln);
      if constexpr (FUSED) {
        u32x4 hw;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float h0 = __fadd_rn(bf16_lo(xv[j]), bf16_lo(rv[j]));
          const float h1 = __fadd_rn(bf16_hi(xv[j]), bf16_hi(rv[j]));
          ss = __fma_rn((double)h0, (double)h0, ss);
          ss = __fma_rn((double)h1, (double)h1, ss);
          hw[j] = pack_bf16x2(h0, h1);
        }
        hb[v] = hw;
        if (in_row(v, ln)) __builtin_nontemporal_store(hw, res_row + v * (kPipeChunk / 8) + ln);
      } else {
        hb[v] = xv;
      }
      __builtin_amdgcn_sched_barrier(0);   // loads stay where they are issued: PIPE chunks in flight
    }
    float rstd = 1.0f;
    if constexpr (FUSED) {
      ss = wave_sum_f64(ss);
      rstd = (float)(1.0 / sqrt(ss / (double)H + (double)a.eps));
    }
#pragma unroll
    for (int v = 0; v < CH; v++) {
      const int e = v * kPipeChunk + ln * 8;
      float y[8];
      if constexpr (FUSED) {
        const u32x4 wv = wl[v * (kPipeChunk / 8) + ln];   // past H: stale LDS, the lane stores nothing
#pragma unroll
        for (int j = 0; j < 4; j++) {
          y[2 * j] = __fmul_rn(__fmul_rn(bf16_lo(hb[v][j]), rstd), bf16_lo(wv[j]));
          y[2 * j + 1] = __fmul_rn(__fmul_rn(bf16_hi(hb[v][j]), rstd), bf16_hi(wv[j]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          y[2 * j] = bf16_lo(hb[v][j]);
          y[2 * j + 1] = bf16_hi(hb[v][j]);
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(y[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
      if constexpr (LPB == 4) amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
      float inv;
      const uint32_t sb = (FMT == kNVFP4) ? nv_block_scale(amax, gs, &inv) : mx_block_scale(amax, &inv);
#pragma unroll
      for (int i = 0; i < 8; i++) y[i] = __fmul_rn(y[i], inv);
      const uint32_t code = e2m1x8(y);
      if (in_row(v, ln)) {
        code_row[v * (kPipeChunk / 8) + ln] = code;
        if (ln % LPB == 0) {
          const int kb = e / B, j = kb & 7;
          const int in_grp = (FMT == kNVFP4) ? ((j >> 2) << 7) + (j & 3)
                                             : (((j >> 1) & 1) << 7) + (j & 1) + ((j >> 2) << 1);
          sf_row[(a.layout == kLinear) ? kb : ((kb >> 3) << 8) + in_grp] = (uint8_t)sb;
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one chunk at a time: keeps the wave's registers few
    }
    if (a.layout == kTiled)
      for (int64_t kb = nblk + ln; kb < (((nblk + 7) >> 3) << 3); kb += kWave)
        a.out_sf[sf_offset(FMT, kTiled, row, kb, nblk)] = 0;
  }
  // TILED: every scale byte of the padding rows M .. rows_grid - 1 is zero
  if (a.layout == kTiled) {
    const int64_t nblk_pad = ((nblk + 7) >> 3) << 3;
    for (int64_t r = a.M + wid; r < a.rows_grid; r += nw)
      for (int64_t kb = lane; kb < nblk_pad; kb += kWave) a.out_sf[sf_offset(FMT, kTiled, r, kb, nblk)] = 0;
  }
}

template <int FMT, int CH, bool FUSED>
hipError_t launch_pipe(const RowArgs& a, hipStream_t s) {
  constexpr int kWavesPerWg = kThreads / kWave;
  int64_t grid = (a.rows_grid + kWavesPerWg - 1) / kWavesPerWg;
  if (grid > (int64_t)kCUs * kPipeWgsPerCu) grid = (int64_t)kCUs * kPipeWgsPerCu;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((row_pipe_kernel<FMT, CH, FUSED>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int FMT, int NBL, int WPR, bool FUSED>
hipError_t launch_row(const RowArgs& a, hipStream_t s) {
  constexpr int ROWS_PER_WG = (kThreads / kWave) / WPR;
  int64_t grid = (a.rows_grid + ROWS_PER_WG - 1) / ROWS_PER_WG;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((row_quant_kernel<FMT, NBL, WPR, FUSED>), dim3((unsigned)grid), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

// Many rows of at most 6144 elements: the pipelined form.  Otherwise pick
// (WPR, NBL) of the row-split form for a row of nblk blocks: one wave per row
// when there are many rows, a row spread over up to 4 waves when there are few.
template <int FMT, bool FUSED>
hipError_t dispatch_row(const RowArgs& a, hipStream_t s) {
  constexpr int MAXNBL = (FMT == kNVFP4) ? 8 : 4;
  const int64_t nblk = a.H / FmtTraits<FMT>::B;
  const int64_t nch = (a.H + kPipeChunk - 1) / kPipeChunk;
  if (a.M >= kPipeMinRows && nch <= kPipeMaxChunks) {
    switch (nch) {
      case 1: return launch_pipe<FMT, 1, FUSED>(a, s);
      case 2: return launch_pipe<FMT, 2, FUSED>(a, s);
      case 3: return launch_pipe<FMT, 3, FUSED>(a, s);
      case 4: return launch_pipe<FMT, 4, FUSED>(a, s);
      case 5: return launch_pipe<FMT, 5, FUSED>(a, s);
      case 6: return launch_pipe<FMT, 6, FUSED>(a, s);
      case 7: return launch_pipe<FMT, 7, FUSED>(a, s);
      case 8: return launch_pipe<FMT, 8, FUSED>(a, s);
      case 9: return launch_pipe<FMT, 9, FUSED>(a, s);
      case 10: return launch_pipe<FMT, 10, FUSED>(a, s);
      case 11: return launch_pipe<FMT, 11, FUSED>(a, s);
      default: return launch_pipe<FMT, 12, FUSED>(a, s);
    }
  }
  int wpr = (a.M >= 1024) ? 1 : 4;
  if (nblk <= 64) wpr = 1;
  while (wpr < 4 && (nblk + 64 * wpr - 1) / (64 * wpr) > MAXNBL) wpr *= 2;
  int64_t nbl = (nblk + 64 * wpr - 1) / (64 * wpr);
  if (nbl > MAXNBL) return hipErrorInvalidValue;
#define LB_CASE(W, N)                                                            \
  if (wpr == W && nbl == N) return launch_row<FMT, N, W, FUSED>(a, s);
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
// Dequantize: one lane per block.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* packed, const uint8_t* sf,
                                                           int64_t rows, int64_t K, int layout,
                                                           const float* gsp, uint16_t* out) {
  constexpr int B = FmtTraits<FMT>::B;
  const int64_t nblk = K / B;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= rows * nblk) return;
  const int64_t row = t / nblk, kb = t % nblk;
  const uint32_t sb = sf[sf_offset(FMT, layout, row, kb, nblk)];
  const float scale = (FMT == kNVFP4) ? e4m3_to_f32(sb) : ue8m0_to_f32(sb);
  const float gs = (FMT == kNVFP4 && gsp != nullptr) ? *gsp : 1.0f;
  const uint8_t* src = packed + row * (K / 2) + kb * (B / 2);
  uint16_t* dst = out + row * K + kb * B;
#pragma unroll
  for (int q = 0; q < B / 16; q++) {
    uint2 p = *reinterpret_cast<const uint2*>(src + q * 8);
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      uint32_t byte = ((j < 4 ? p.x : p.y) >> (8 * (j & 3))) & 0xFF;
      float v0 = __fmul_rn(e2m1_to_f32(byte & 15), scale);   // exact
      float v1 = __fmul_rn(e2m1_to_f32(byte >> 4), scale);
      if (FMT == kNVFP4) { v0 = __fdiv_rn(v0, gs); v1 = __fdiv_rn(v1, gs); }
      o[j] = pack_bf16x2(v0, v1);
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst + q * 16);
    d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

}  // namespace

hipError_t launch_add_rmsnorm_quant(const uint16_t* x, uint16_t* residual, const uint16_t* w, int64_t M,
                                    int64_t H, float eps, int fmt, int layout, const float* gs,
                                    uint8_t* out_packed, uint8_t* out_sf, hipStream_t s) {
  RowArgs a{x, residual, w, M, H, M, eps, layout, gs, out_packed, out_sf};
  if (layout == kTiled) a.rows_grid = (M + 31) / 32 * 32;
  return fmt == kNVFP4 ? dispatch_row<kNVFP4, true>(a, s) : dispatch_row<kMXFP4, true>(a, s);
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t K, int fmt, int layout,
                           const float* gs, uint8_t* out_packed, uint8_t* out_sf, hipStream_t s) {
  RowArgs a{x, nullptr, nullptr, rows, K, rows, 0.0f, layout, gs, out_packed, out_sf};
  if (layout == kTiled) a.rows_grid = (rows + 31) / 32 * 32;
  return fmt == kNVFP4 ? dispatch_row<kNVFP4, false>(a, s) : dispatch_row<kMXFP4, false>(a, s);
}

hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K, int fmt,
                             int layout, const float* gs, uint16_t* out, hipStream_t s) {
  const int64_t nblk = K / (fmt == kNVFP4 ? 16 : 32);
  const int64_t n = rows * nblk;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
  if (fmt == kNVFP4)
    hipLaunchKernelGGL(dequant_kernel<kNVFP4>, dim3(grid), dim3(kThreads), 0, s, packed, sf, rows, K, layout,
                       gs, out);
  else
    hipLaunchKernelGGL(dequant_kernel<kMXFP4>, dim3(grid), dim3(kThreads), 0, s, packed, sf, rows, K, layout,
                       gs, out);
  return hipGetLastError();
}

}  // namespace lowbit
