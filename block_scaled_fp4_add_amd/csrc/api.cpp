// api.cpp -- the extern "C" entry points of liblowbit.so: argument checks,
// device check, schedule choice, launch.  Declared and documented in
// include/lowbit.h.
//
// Checks run in a fixed order -- enums and pointers (EINVAL), sizes (ESHAPE),
// alignment (EALIGN), then the device (EDEVICE) -- and nothing is launched
// unless all pass.  The device query happens last, so every argument error is
// reported the same way with or without a GPU present.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"
#include "lowbit.h"

// Split-K workspace of lowbit_gemm_bf16_noalloc: a file-scope device array,
// one copy per device, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device memory: its device address is
// looked up per device with hipGetSymbolAddress and only that address is
// handed to kernels.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static_assert(kStaticScratchBytes == LOWBIT_STATIC_SCRATCH_BYTES, "header and library disagree");
static_assert((int)LOWBIT_MXFP8_MMA == (int)lowbit::kMXFP8Mma && (int)LOWBIT_MXFP8 == (int)lowbit::kMXFP8, "format ids");
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {

using lowbit::GemmArgs;

constexpr int64_t kMaxRowElems = 32768;  // 4 waves x 64 lanes x 128 elements per lane

// GEMM operand formats (MXFP8 operands take LINEAR scales only)
bool fmt_ok(int f) { return f == LOWBIT_NVFP4 || f == LOWBIT_MXFP4 || f == LOWBIT_MXFP8 || f == LOWBIT_MXFP8_MMA; }
// MXFP8 operands, exact or on the scaled FP8 MFMA
bool fp8_fmt(int f) { return f == LOWBIT_MXFP8 || f == LOWBIT_MXFP8_MMA; }
bool fp4_fmt(int f) { return f == LOWBIT_NVFP4 || f == LOWBIT_MXFP4; }
bool layout_ok(int l) { return l == LOWBIT_SF_LINEAR || l == LOWBIT_SF_TILED; }
bool gemm_layout_ok(int f, int l) { return fp8_fmt(f) ? l == LOWBIT_SF_LINEAR : layout_ok(l); }
// packed bytes of a row of k elements: one per MXFP8 element, else two codes a byte
int64_t packed_row_bytes(int f, int64_t k) { return fp8_fmt(f) ? k : k / 2; }
// producer / quantizer / dequantizer: MXFP8 and 32-block NVFP4 as well, with
// LINEAR scales only; the FP4 GEMM formats also take the 128 x 4 swizzle
bool qfmt_layout_ok(int f, int l) {
  if (f == LOWBIT_MXFP8 || f == LOWBIT_NVFP4_B32) return l == LOWBIT_SF_LINEAR;
  return fp4_fmt(f) && (layout_ok(l) || l == LOWBIT_SF_SWZ128);
}

int64_t block_of(int f) { return f == LOWBIT_NVFP4 ? 16 : 32; }
// formats with E4M3 block scales, the only ones that take a global scale
bool takes_gs(int f) { return f == LOWBIT_NVFP4 || f == LOWBIT_NVFP4_B32; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// gfx950 check, cached per device ordinal.
lowbit_status device_check() {
  static std::mutex mu;
  static int cached[64];  // 0 unknown, 1 ok, 2 not gfx950
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return LOWBIT_EDEVICE;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
      (void)hipGetLastError();
      return LOWBIT_EDEVICE;
    }
    cached[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  return cached[dev] == 1 ? LOWBIT_OK : LOWBIT_EDEVICE;
}

lowbit_status from_hip(hipError_t e) { return e == hipSuccess ? LOWBIT_OK : LOWBIT_EHIP; }

// Device address of `scratch` on the current device, resolved on the first
// call on that device (with it current) and kept per device.
lowbit_status static_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return LOWBIT_EHIP;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return LOWBIT_EHIP;
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return LOWBIT_OK;
}

lowbit_status check_sf_ptr(const void* sf, int layout) {
  if (layout == LOWBIT_SF_TILED && !aligned(sf, 4)) return LOWBIT_EALIGN;
  return LOWBIT_OK;
}

lowbit_status gemm_common(const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                          int64_t M, int64_t N, int64_t K, int fmt, int la, int lb, float alpha,
                          int epi, const void* bias, const void* residual, void* out,
                          const float* gs_out, uint8_t* out_packed, uint8_t* out_sf, int out_layout,
                          int variant, void* workspace, size_t workspace_bytes, hipStream_t stream,
                          bool static_ws = false) {
  const bool fp4_out = epi == lowbit::kEpiBiasGeluFp4;
  const bool fp8_out = epi == lowbit::kEpiFp8;
  const bool q_out = fp4_out || fp8_out;   // packed output plus scales
  // EINVAL: enums and pointers
  if (!fmt_ok(fmt) || !gemm_layout_ok(fmt, la) || !gemm_layout_ok(fmt, lb)) return LOWBIT_EINVAL;
  if (fp4_out && !layout_ok(out_layout)) return LOWBIT_EINVAL;
  if (fp4_out && fp8_fmt(fmt)) return LOWBIT_EINVAL;   // NVFP4 output from FP4 operands only
  if (fp8_out && out_layout != LOWBIT_SF_LINEAR && out_layout != LOWBIT_SF_SWZ128) return LOWBIT_EINVAL;
  if (variant < -1 || variant > lowbit::kVariantSplitK) return LOWBIT_EINVAL;
  if (workspace_bytes > 0 && !workspace) return LOWBIT_EINVAL;
  if (M < 0 || N < 0 || K < 0) return LOWBIT_ESHAPE;
  const bool empty = (M == 0 || N == 0);
  if (!empty) {
    if (!a || !b || !sfa || !sfb) return LOWBIT_EINVAL;
    const bool needs_bias = epi == lowbit::kEpiBias || epi == lowbit::kEpiBiasResidual ||
                            epi == lowbit::kEpiBiasGelu || fp4_out;
    const bool needs_res = epi == lowbit::kEpiResidual || epi == lowbit::kEpiBiasResidual;
    if (needs_bias && !bias) return LOWBIT_EINVAL;
    if (needs_res && !residual) return LOWBIT_EINVAL;
    if (q_out ? (!out_packed || !out_sf) : !out) return LOWBIT_EINVAL;
  }
  // ESHAPE
  const int64_t B = block_of(fmt);
  if (K < B || K % B != 0) return LOWBIT_ESHAPE;
  if (fp4_out && N % 16 != 0) return LOWBIT_ESHAPE;
  if (fp8_out && N % 32 != 0) return LOWBIT_ESHAPE;
  // workspace on offer: the caller's, or the static scratch
  const size_t ws_avail = static_ws ? kStaticScratchBytes : (workspace ? workspace_bytes : 0);
  int v = lowbit::gemm_pick_variant(M, N, K, fmt, variant, ws_avail);
  if (v < 0) return LOWBIT_ESHAPE;
  // split-K asked for explicitly needs the workspace it documents; beyond
  // the static scratch that is a size the entry point does not take
  const lowbit::SplitPlan plan = lowbit::gemm_splitk_plan(M, N, K, fmt, variant == lowbit::kVariantSplitK);
  if (v == lowbit::kVariantSplitK && !empty && ws_avail < plan.bytes)
    return static_ws ? LOWBIT_ESHAPE : LOWBIT_EINVAL;
  // the 128 x 384 schedule reads LINEAR scales as aligned words: an automatic
  // split on it falls back to the unsplit schedule, an explicit one is refused
  if (v == lowbit::kVariantSplitK && plan.nv &&
      ((la == LOWBIT_SF_LINEAR && !aligned(sfa, 4)) || (lb == LOWBIT_SF_LINEAR && !aligned(sfb, 4)))) {
    if (variant == lowbit::kVariantSplitK) return LOWBIT_EALIGN;
    v = lowbit::gemm_pick_variant(M, N, K, fmt, variant, 0);
  }
  // the prefill schedules (and the split of the 128 x 384 one) address each
  // operand through a 32-bit buffer offset
  if ((v == 1 || (v == lowbit::kVariantSplitK && plan.nv)) &&
      (M * packed_row_bytes(fmt, K) >= (int64_t(1) << 30) || N * packed_row_bytes(fmt, K) >= (int64_t(1) << 30)))
    return LOWBIT_ESHAPE;
  if (empty) return LOWBIT_OK;
  // EALIGN
  if (!aligned(a, 16) || !aligned(b, 16)) return LOWBIT_EALIGN;
  if (check_sf_ptr(sfa, la) || check_sf_ptr(sfb, lb)) return LOWBIT_EALIGN;
  if (bias && !aligned(bias, 16)) return LOWBIT_EALIGN;
  if (residual && !aligned(residual, 16)) return LOWBIT_EALIGN;
  if (fp4_out) {
    if (!aligned(out_packed, 8) || (out_layout == LOWBIT_SF_TILED && !aligned(out_sf, 4)))
      return LOWBIT_EALIGN;
    if (gs_out && !aligned(gs_out, 4)) return LOWBIT_EALIGN;
  } else if (fp8_out) {
    if (!aligned(out_packed, 16)) return LOWBIT_EALIGN;
  } else if (!aligned(out, 16)) {
    return LOWBIT_EALIGN;
  }
  if (v == lowbit::kVariantSplitK && !static_ws && !aligned(workspace, 16)) return LOWBIT_EALIGN;
  // EDEVICE
  if (lowbit_status d = device_check()) return d;
  if (v == lowbit::kVariantSplitK && static_ws) {
    if (lowbit_status e = static_scratch(&workspace)) return e;
  }
  GemmArgs g{};
  g.a = a;
  g.b = b;
  g.sfa = sfa;
  g.sfb = sfb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.fmt = fmt == LOWBIT_MXFP8_MMA ? LOWBIT_MXFP8 : fmt;   // the kernels run MXFP8 operands either way
  g.f8mma = fmt == LOWBIT_MXFP8_MMA ? 1 : 0;
  g.la = la;
  g.lb = lb;
  g.alpha = alpha;
  g.epi = epi;
  g.bias = static_cast<const uint16_t*>(bias);
  g.residual = static_cast<const uint16_t*>(residual);
  g.out = static_cast<uint16_t*>(out);
  g.gs_out = gs_out;
  g.out_packed = out_packed;
  g.out_sf = out_sf;
  g.out_layout = out_layout;
  if (v == lowbit::kVariantSplitK) {
    g.ws = static_cast<float*>(workspace);
    g.splits = plan.splits;
    g.per = plan.per;
    g.split_nv = plan.nv ? 1 : 0;
  }
  if (getenv("LOWBIT_LOG"))
    fprintf(stderr, "[lowbit] gemm M=%lld N=%lld K=%lld fmt=%d epi=%d variant=%d\n", (long long)M,
            (long long)N, (long long)K, fmt, epi, v);
  return from_hip(lowbit::launch_gemm(g, v, stream));
}

static lowbit_status producer(const void* input, void* residual, const void* weight, int64_t M, int64_t H,
                              float eps, lowbit_format fmt, lowbit_sf_layout layout, const float* global_scale,
                              uint8_t* out_packed, uint8_t* out_sf, uint8_t* out_sf_lin, int in_f16,
                              hipStream_t stream) {
  if (!qfmt_layout_ok(fmt, layout)) return LOWBIT_EINVAL;
  if (!takes_gs(fmt) && global_scale) return LOWBIT_EINVAL;
  // the second copy of the scales sits beside a padded layout of an FP4 format
  if (out_sf_lin && (!fp4_fmt(fmt) || (layout != LOWBIT_SF_TILED && layout != LOWBIT_SF_SWZ128)))
    return LOWBIT_EINVAL;
  if (M < 0) return LOWBIT_ESHAPE;
  if (M > 0 && (!input || !residual || !weight || !out_packed || !out_sf)) return LOWBIT_EINVAL;
  if (H < 64 || H % block_of(fmt) != 0 || H > kMaxRowElems) return LOWBIT_ESHAPE;
  if (M == 0) return LOWBIT_OK;
  if (!aligned(input, 16) || !aligned(residual, 16) || !aligned(weight, 16) || !aligned(out_packed, 16))
    return LOWBIT_EALIGN;
  if (check_sf_ptr(out_sf, layout) || (global_scale && !aligned(global_scale, 4))) return LOWBIT_EALIGN;
  if (lowbit_status d = device_check()) return d;
  return from_hip(lowbit::launch_add_rmsnorm_quant(
      static_cast<const uint16_t*>(input), static_cast<uint16_t*>(residual),
      static_cast<const uint16_t*>(weight), M, H, eps, fmt, layout, global_scale, out_packed, out_sf,
      out_sf_lin, in_f16, stream));
}

static lowbit_status quantize(const void* x, int64_t rows, int64_t K, lowbit_format fmt, lowbit_sf_layout layout,
                              const float* global_scale, uint8_t* out_packed, uint8_t* out_sf, int in_f16,
                              hipStream_t stream) {
  if (!qfmt_layout_ok(fmt, layout)) return LOWBIT_EINVAL;
  if (!takes_gs(fmt) && global_scale) return LOWBIT_EINVAL;
  if (rows < 0) return LOWBIT_ESHAPE;
  if (rows > 0 && (!x || !out_packed || !out_sf)) return LOWBIT_EINVAL;
  if (K < block_of(fmt) || K % block_of(fmt) != 0 || K > kMaxRowElems) return LOWBIT_ESHAPE;
  if (rows == 0) return LOWBIT_OK;
  if (!aligned(x, 16) || !aligned(out_packed, 16)) return LOWBIT_EALIGN;
  if (check_sf_ptr(out_sf, layout) || (global_scale && !aligned(global_scale, 4))) return LOWBIT_EALIGN;
  if (lowbit_status d = device_check()) return d;
  return from_hip(lowbit::launch_quantize(static_cast<const uint16_t*>(x), rows, K, fmt, layout,
                                          global_scale, out_packed, out_sf, in_f16, stream));
}

static lowbit_status dequantize(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K, int fmt,
                                int layout, const float* global_scale, void* out, int out_f16,
                                hipStream_t stream) {
  if (!qfmt_layout_ok(fmt, layout)) return LOWBIT_EINVAL;
  if (!takes_gs(fmt) && global_scale) return LOWBIT_EINVAL;
  if (rows < 0) return LOWBIT_ESHAPE;
  if (rows > 0 && (!packed || !sf || !out)) return LOWBIT_EINVAL;
  if (K < block_of(fmt) || K % block_of(fmt) != 0) return LOWBIT_ESHAPE;
  if (rows == 0) return LOWBIT_OK;
  if (!aligned(packed, 16) || !aligned(out, 16)) return LOWBIT_EALIGN;
  if (global_scale && !aligned(global_scale, 4)) return LOWBIT_EALIGN;
  if (lowbit_status d = device_check()) return d;
  return from_hip(lowbit::launch_dequantize(packed, sf, rows, K, fmt, layout, global_scale,
                                            static_cast<uint16_t*>(out), out_f16, stream));
}

}  // namespace

extern "C" {

const char* lowbit_status_str(lowbit_status s) {
  switch (s) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_EINVAL: return "invalid argument";
    case LOWBIT_EALIGN: return "misaligned pointer";
    case LOWBIT_ESHAPE: return "unsupported shape";
    case LOWBIT_EDEVICE: return "device is not gfx950";
    case LOWBIT_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t lowbit_sf_bytes(int64_t rows, int64_t k, lowbit_format fmt, lowbit_sf_layout layout) {
  // the quantization formats and layouts, and the FP8 GEMM output's 128 x 4 layout
  // (LOWBIT_MXFP8_MMA: the MXFP8 scale bytes it reads)
  if (fmt == LOWBIT_MXFP8_MMA) fmt = LOWBIT_MXFP8;
  const bool ok = qfmt_layout_ok(fmt, layout) || (fmt == LOWBIT_MXFP8 && layout == LOWBIT_SF_SWZ128);
  if (!ok || rows < 0 || k < 0 || k % block_of(fmt) != 0) return 0;
  return (size_t)lowbit::sf_bytes_of(layout, rows, k / block_of(fmt));
}

lowbit_status lowbit_add_rmsnorm_quant(const void* input, void* residual, const void* weight, int64_t M,
                                       int64_t H, float eps, lowbit_format fmt, lowbit_sf_layout layout,
                                       const float* global_scale, uint8_t* out_packed, uint8_t* out_sf,
                                       hipStream_t stream) {
  return producer(input, residual, weight, M, H, eps, fmt, layout, global_scale, out_packed, out_sf, nullptr,
                  0, stream);
}

lowbit_status lowbit_add_rmsnorm_quant_fp16(const void* input, void* residual, const void* weight, int64_t M,
                                            int64_t H, float eps, lowbit_format fmt, lowbit_sf_layout layout,
                                            const float* global_scale, uint8_t* out_packed, uint8_t* out_sf,
                                            hipStream_t stream) {
  return producer(input, residual, weight, M, H, eps, fmt, layout, global_scale, out_packed, out_sf, nullptr,
                  1, stream);
}

lowbit_status lowbit_add_rmsnorm_quant_both_sf(const void* input, void* residual, const void* weight, int64_t M,
                                               int64_t H, float eps, lowbit_format fmt, lowbit_sf_layout layout,
                                               const float* global_scale, uint8_t* out_packed, uint8_t* out_sf,
                                               uint8_t* out_sf_linear, hipStream_t stream) {
  if (M > 0 && !out_sf_linear) return LOWBIT_EINVAL;
  return producer(input, residual, weight, M, H, eps, fmt, layout, global_scale, out_packed, out_sf,
                  out_sf_linear, 0, stream);
}

lowbit_status lowbit_add_rmsnorm_quant_both_sf_fp16(const void* input, void* residual, const void* weight,
                                                    int64_t M, int64_t H, float eps, lowbit_format fmt,
                                                    lowbit_sf_layout layout, const float* global_scale,
                                                    uint8_t* out_packed, uint8_t* out_sf, uint8_t* out_sf_linear,
                                                    hipStream_t stream) {
  if (M > 0 && !out_sf_linear) return LOWBIT_EINVAL;
  return producer(input, residual, weight, M, H, eps, fmt, layout, global_scale, out_packed, out_sf,
                  out_sf_linear, 1, stream);
}

lowbit_status lowbit_quantize(const void* x, int64_t rows, int64_t K, lowbit_format fmt,
                              lowbit_sf_layout layout, const float* global_scale, uint8_t* out_packed,
                              uint8_t* out_sf, hipStream_t stream) {
  return quantize(x, rows, K, fmt, layout, global_scale, out_packed, out_sf, 0, stream);
}

lowbit_status lowbit_quantize_fp16(const void* x, int64_t rows, int64_t K, lowbit_format fmt,
                                   lowbit_sf_layout layout, const float* global_scale, uint8_t* out_packed,
                                   uint8_t* out_sf, hipStream_t stream) {
  return quantize(x, rows, K, fmt, layout, global_scale, out_packed, out_sf, 1, stream);
}

lowbit_status lowbit_rope_quant(const void* x, const int64_t* positions, const float* rope, int64_t T,
                                int64_t heads, int64_t D, int64_t R, int64_t P, lowbit_format fmt,
                                lowbit_sf_layout layout, uint8_t* out_packed, uint8_t* out_sf,
                                hipStream_t stream) {
  // EINVAL: formats (MXFP8 with LINEAR scales, MXFP4 with any FP4 layout) and pointers
  if (fmt != LOWBIT_MXFP8 && fmt != LOWBIT_MXFP4) return LOWBIT_EINVAL;
  if (!qfmt_layout_ok(fmt, layout)) return LOWBIT_EINVAL;
  const bool empty = T == 0;
  if (!empty && (!x || !out_packed || !out_sf)) return LOWBIT_EINVAL;
  if (!empty && R > 0 && (!positions || !rope)) return LOWBIT_EINVAL;
  // ESHAPE
  if (T < 0 || heads < 1 || D < 32 || D % 32 != 0 || D > kMaxRowElems) return LOWBIT_ESHAPE;
  if (R < 0 || R > D || R % 2 != 0 || (R > 0 && P < 1)) return LOWBIT_ESHAPE;
  // the kernel indexes 8-element units in 32 bits (rows padded to 128 at most)
  if (T > 0 && ((T * heads + 127) / 128 * 128) * (D / 8) >= (int64_t(1) << 31)) return LOWBIT_ESHAPE;
  if (empty) return LOWBIT_OK;
  // EALIGN
  if (!aligned(x, 16) || !aligned(out_packed, 16)) return LOWBIT_EALIGN;
  if (R > 0 && (!aligned(positions, 8) || !aligned(rope, 4))) return LOWBIT_EALIGN;
  if (lowbit_status d = device_check()) return d;
  lowbit::RopeArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.positions = positions;
  a.rope = rope;
  a.rows = T * heads;
  a.heads = heads;
  a.D = D;
  a.R = R;
  a.P = P;
  a.out_packed = out_packed;
  a.out_sf = out_sf;
  return from_hip(lowbit::launch_rope_quant(a, fmt, layout, stream));
}

lowbit_status lowbit_dequantize(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K,
                                lowbit_format fmt, lowbit_sf_layout layout, const float* global_scale,
                                void* out, hipStream_t stream) {
  return dequantize(packed, sf, rows, K, fmt, layout, global_scale, out, 0, stream);
}

lowbit_status lowbit_dequantize_fp16(const uint8_t* packed, const uint8_t* sf, int64_t rows, int64_t K,
                                     lowbit_format fmt, lowbit_sf_layout layout, const float* global_scale,
                                     void* out, hipStream_t stream) {
  return dequantize(packed, sf, rows, K, fmt, layout, global_scale, out, 1, stream);
}

lowbit_status lowbit_sf_convert(const uint8_t* src, lowbit_sf_layout src_layout, uint8_t* dst,
                                lowbit_sf_layout dst_layout, int64_t rows, int64_t k, lowbit_format fmt,
                                hipStream_t stream) {
  // every (format, layout) pair that has a scale buffer size
  if (lowbit_sf_bytes(1, block_of(fmt), fmt, src_layout) == 0 ||
      lowbit_sf_bytes(1, block_of(fmt), fmt, dst_layout) == 0)
    return LOWBIT_EINVAL;
  if (rows < 0) return LOWBIT_ESHAPE;
  if (rows > 0 && (!src || !dst)) return LOWBIT_EINVAL;
  if (k < block_of(fmt) || k % block_of(fmt) != 0) return LOWBIT_ESHAPE;
  if (rows == 0) return LOWBIT_OK;
  const size_t sbytes = lowbit_sf_bytes(rows, k, fmt, src_layout);
  const size_t dbytes = lowbit_sf_bytes(rows, k, fmt, dst_layout);
  if ((int64_t)dbytes > lowbit::kRelayoutMaxBytes) return LOWBIT_ESHAPE;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + dbytes && d0 < s0 + sbytes) return LOWBIT_EINVAL;   // the buffers overlap
  if (lowbit_status d = device_check()) return d;
  return from_hip(lowbit::launch_sf_relayout(src, src_layout, dst, dst_layout, rows, k / block_of(fmt), fmt,
                                             stream));
}

lowbit_status lowbit_gemm_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                               int64_t M, int64_t N, int64_t K, lowbit_format fmt,
                               lowbit_sf_layout sfa_layout, lowbit_sf_layout sfb_layout, float alpha,
                               void* out, int variant, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha, lowbit::kEpiNone,
                     nullptr, nullptr, out, nullptr, nullptr, nullptr, 0, variant, workspace, workspace_bytes,
                     stream);
}

lowbit_status lowbit_gemm_bf16_noalloc(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                       const uint8_t* sfb, int64_t M, int64_t N, int64_t K, lowbit_format fmt,
                                       lowbit_sf_layout sfa_layout, lowbit_sf_layout sfb_layout, float alpha,
                                       void* out, int variant, hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha, lowbit::kEpiNone,
                     nullptr, nullptr, out, nullptr, nullptr, nullptr, 0, variant, nullptr, 0, stream, true);
}

lowbit_status lowbit_gemm_bias_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                    const uint8_t* sfb, int64_t M, int64_t N, int64_t K, lowbit_format fmt,
                                    lowbit_sf_layout sfa_layout, lowbit_sf_layout sfb_layout, float alpha,
                                    const void* bias, void* out, int variant, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha, lowbit::kEpiBias, bias,
                     nullptr, out, nullptr, nullptr, nullptr, 0, variant, workspace, workspace_bytes, stream);
}

lowbit_status lowbit_gemm_residual_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                        const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                        lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                        lowbit_sf_layout sfb_layout, float alpha, const void* residual,
                                        void* out, int variant, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha, lowbit::kEpiResidual,
                     nullptr, residual, out, nullptr, nullptr, nullptr, 0, variant, workspace, workspace_bytes,
                     stream);
}

lowbit_status lowbit_gemm_bias_residual_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                             const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                             lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                             lowbit_sf_layout sfb_layout, float alpha, const void* bias,
                                             const void* residual, void* out, int variant, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha,
                     lowbit::kEpiBiasResidual, bias, residual, out, nullptr, nullptr, nullptr, 0, variant,
                     workspace, workspace_bytes, stream);
}

lowbit_status lowbit_gemm_bias_gelu_bf16(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                         const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                         lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                         lowbit_sf_layout sfb_layout, float alpha, const void* bias,
                                         void* out, int variant, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha, lowbit::kEpiBiasGelu,
                     bias, nullptr, out, nullptr, nullptr, nullptr, 0, variant, workspace, workspace_bytes,
                     stream);
}

lowbit_status lowbit_gemm_fp8(const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                              int64_t M, int64_t N, int64_t K, lowbit_format fmt, lowbit_sf_layout sfa_layout,
                              lowbit_sf_layout sfb_layout, float alpha, uint8_t* out_packed, uint8_t* out_sf,
                              lowbit_sf_layout out_layout, int variant, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha, lowbit::kEpiFp8, nullptr,
                     nullptr, nullptr, nullptr, out_packed, out_sf, out_layout, variant, workspace,
                     workspace_bytes, stream);
}

lowbit_status lowbit_gemm_bias_gelu_fp4(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                        const uint8_t* sfb, int64_t M, int64_t N, int64_t K,
                                        lowbit_format fmt, lowbit_sf_layout sfa_layout,
                                        lowbit_sf_layout sfb_layout, float alpha, const void* bias,
                                        const float* out_global_scale, uint8_t* out_packed,
                                        uint8_t* out_sf, lowbit_sf_layout out_layout, int variant,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gemm_common(a, b, sfa, sfb, M, N, K, fmt, sfa_layout, sfb_layout, alpha,
                     lowbit::kEpiBiasGeluFp4, bias, nullptr, nullptr, out_global_scale, out_packed, out_sf,
                     out_layout, variant, workspace, workspace_bytes, stream);
}

int lowbit_gemm_pick_variant(int64_t M, int64_t N, int64_t K, lowbit_format fmt, int variant,
                             size_t workspace_bytes) {
  if (!fmt_ok(fmt) || M < 0 || N < 0 || K < block_of(fmt) || K % block_of(fmt) != 0) return -1;
  if (variant < -1 || variant > lowbit::kVariantSplitK) return -1;
  return lowbit::gemm_pick_variant(M, N, K, fmt, variant, workspace_bytes);
}

size_t lowbit_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, lowbit_format fmt, int variant) {
  if (!fmt_ok(fmt) || M < 0 || N < 0 || K < block_of(fmt) || K % block_of(fmt) != 0) return 0;
  if (variant != -1 && variant != lowbit::kVariantSplitK) return 0;
  return lowbit::gemm_splitk_plan(M, N, K, fmt, variant == lowbit::kVariantSplitK).bytes;
}

}  // extern "C"
