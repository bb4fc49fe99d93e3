// launch.hpp -- internal launchers behind the C ABI (arguments already
// validated by api.cpp; every pointer is a device pointer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

// in_f16: the 16-bit input tensors (x, residual, weight) are fp16, else bf16.
// out_sf_lin: nullptr, or (with layout TILED) a second scale buffer that gets
// the same bytes in the LINEAR layout.
hipError_t launch_add_rmsnorm_quant(const uint16_t* x, uint16_t* residual, const uint16_t* w, int64_t M,
                                    int64_t H, float eps, int fmt, int layout, const float* gs,
                                    uint8_t* out_packed, uint8_t* out_sf, uint8_t* out_sf_lin, int in_f16,
                                    hipStream_t s);

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t K, int fmt, int layout,
                           const float* gs, uint8_t* out_packed, uint8_t* out_sf, int in_f16, hipStream_t s);

// out: bf16, or fp16 with out_f16
hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K, int fmt,
                             int layout, const float* gs, uint16_t* out, int out_f16, hipStream_t s);

// Scale bytes of a (rows, nblk blocks) operand rewritten from layout ls into
// layout ld, destination padding zero; at most kRelayoutMaxBytes of output.
constexpr int64_t kRelayoutMaxBytes = int64_t(1) << 33;
hipError_t launch_sf_relayout(const uint8_t* src, int ls, uint8_t* dst, int ld, int64_t rows, int64_t nblk,
                              int fmt, hipStream_t s);

// Inverse RoPE + MX quantization of (T, heads, D) bf16 rows (rows = T * heads).
struct RopeArgs {
  const uint16_t* x;          // bf16 (rows, D)
  const int64_t* positions;   // (T) table rows; nullptr when R == 0
  const float* rope;          // fp32 (P, R): cos || sin per row; nullptr when R == 0
  int64_t rows, heads, D, R, P;
  int64_t rows_grid;          // rows the grid covers (padded scale layouts pad the rows)
  uint8_t* out_packed;        // MXFP8 (rows, D) / MXFP4 (rows, D/2)
  uint8_t* out_sf;
};
hipError_t launch_rope_quant(const RopeArgs& a, int fmt, int layout, hipStream_t s);

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* b;
  const uint8_t* sfa;
  const uint8_t* sfb;
  int64_t M, N, K;
  int fmt;
  int la, lb;                 // scale layouts of A and B
  float alpha;
  int epi;                    // Epi
  const uint16_t* bias;       // (N) or nullptr
  const uint16_t* residual;   // (M, N) or nullptr
  uint16_t* out;              // bf16 (M, N)
  const float* gs_out;        // FP4 output: global scale or nullptr
  uint8_t* out_packed;        // FP4 output: (M, N/2); FP8 output: (M, N)
  uint8_t* out_sf;            // FP4 / FP8 output scales
  int out_layout;
  float* ws;                  // split-K: fp32 partial tiles (device), else nullptr
  int splits;                 // split-K: workgroups along K per output tile
  int per;                    // split-K: K units per split (supersteps, or the stages of split_nv)
  int split_nv;               // split-K on a prefill schedule: 128 x 384 (units: its 64-byte row stages),
                              // or with f8mma 256 x 256 (units: its supersteps of 128 elements)
  int f8mma;                  // MXFP8 operands on the scaled FP8 MFMA (kMXFP8Mma), else exact bf16 dequantization
};

// Schedules: 0 decode, 1 prefill, 2 split-K decode (needs a workspace).
constexpr int kVariantSplitK = 2;

// Split-K plan of a GEMM: `splits` workgroups along K per output tile (1: no
// split), `per` K units each, `bytes` of workspace for the partials.  force:
// at least two splits whenever K has two units.  nv: a prefill schedule does
// the partial pass -- NVFP4 with 64 < M <= 128 and K % 64 == 0, and above 128
// rows NVFP4 (K % 64 == 0) or MXFP8 (K % 128 == 0), on the 128 x 384 tiles
// (units: stages of 64 bytes of a row, 128 NVFP4 or 64 MXFP8 elements);
// above 128 rows kMXFP8Mma (K % 128 == 0) on the 256 x 256 tiles (units:
// supersteps of 128 elements); above 128 rows only for shapes with at most
// 128 such tiles.  Else the decode schedule (M <= 128, units of one
// superstep).  Either way the partials are 32 x 32 fp32 tiles in one layout,
// summed by the same reduce pass.  fmt: a GEMM format, kMXFP8Mma included.
struct SplitPlan {
  int splits;
  int per;
  size_t bytes;
  bool nv;
};
SplitPlan gemm_splitk_plan(int64_t M, int64_t N, int64_t K, int fmt, bool force);

// Schedule resolution shared by the launcher, lowbit_gemm_pick_variant and
// lowbit_gemm_workspace_bytes: -1 resolves by shape and by the workspace the
// caller offers (ws_bytes); returns -1 for a variant that cannot run the shape.
int gemm_pick_variant(int64_t M, int64_t N, int64_t K, int fmt, int variant, size_t ws_bytes);
hipError_t launch_gemm(const GemmArgs& g, int variant, hipStream_t s);

}  // namespace lowbit
