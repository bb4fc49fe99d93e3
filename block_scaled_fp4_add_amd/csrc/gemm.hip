// gemm.hip -- dispatch of the block-scaled A4W4 GEMM: schedule choice and
// the (format, epilogue) switch over the launchers that the gemm_inst_*.hip
// units instantiate from gemm_kernels.hpp (split so that they compile in
// parallel).
#include "launch.hpp"
#include "common.hpp"

namespace lowbit {
namespace gk {
template <int FMT, int EPI>
hipError_t launch_fmt_epi(const GemmArgs& g, int variant, hipStream_t s);
template <int FMT, int EPI>
hipError_t launch_splitk(const GemmArgs& g, hipStream_t s);
}  // namespace gk

namespace {
using gk::launch_fmt_epi;

template <int FMT, int EPI>
hipError_t launch_one(const GemmArgs& g, int variant, hipStream_t s) {
  return variant == kVariantSplitK ? gk::launch_splitk<FMT, EPI>(g, s) : launch_fmt_epi<FMT, EPI>(g, variant, s);
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& g, int variant, hipStream_t s) {
  switch (g.epi) {
    case kEpiNone: return launch_one<FMT, kEpiNone>(g, variant, s);
    case kEpiBias: return launch_one<FMT, kEpiBias>(g, variant, s);
    case kEpiResidual: return launch_one<FMT, kEpiResidual>(g, variant, s);
    case kEpiBiasResidual: return launch_one<FMT, kEpiBiasResidual>(g, variant, s);
    case kEpiBiasGelu: return launch_one<FMT, kEpiBiasGelu>(g, variant, s);
    case kEpiBiasGeluFp4: return launch_one<FMT, kEpiBiasGeluFp4>(g, variant, s);
    case kEpiFp8: return launch_one<FMT, kEpiFp8>(g, variant, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Split-K targets twice as many workgroups as the chip has CUs, each split
// holding at least four supersteps of K (one per wave; a superstep is 256
// FP4 or 128 FP8 elements).  Its second launch
// costs about as much as one round trip of loads, so the automatic choice
// splits only K of 16 supersteps or more (measured: (41, 1536, 6144) MXFP4
// 13.7 -> 10.7 us split; (41, 4608, 1536) 6.8 -> 9.4 us, so not split).
constexpr int64_t kSplitTargetWorkgroups = 512;
constexpr int64_t kSplitMinSupersteps = 16;
// the 128 x 384 split: one workgroup a CU (256 CUs)
constexpr int64_t kSplitNvWorkgroups = 256;
// more than 128 rows: at least 16 stages a split (the partial tiles then
// cost a few percent of the contraction)
constexpr int64_t kSplitNvMinStagesPrefill = 16;

SplitPlan gemm_splitk_plan(int64_t M, int64_t N, int64_t K, int fmt_in, bool force) {
  // MXFP8 on the scaled FP8 MFMA splits as exact MXFP8 does
  const int fmt = fmt_in == kMXFP8Mma ? kMXFP8 : fmt_in;
  const int64_t ss = fmt == kMXFP8 ? 128 : 256;   // K elements of a superstep
  const int64_t nss = (K + ss - 1) / ss;
  SplitPlan none{1, (int)nss, 0, false};
  if (M <= 0 || N <= 0 || K <= 0) return none;
  const int64_t tiles = (N + 31) / 32, mt = (M + 31) / 32;
  if (M > 128) {
    // Prefill shapes with at most half the CUs' worth of prefill tiles (few
    // columns, long K): the prefill schedule split along K, about one
    // workgroup per CU.  NVFP4 with K % 64 == 0 on the 128 x 384 tiles (units:
    // stages of 128 elements, at least 16 a split); MXFP8 (exact or on the
    // scaled FP8 MFMA) with K % 128 == 0 on the 256 x 256 tiles (units:
    // supersteps of 128 elements, at least 8 a split).  Other formats and
    // shapes do not split.
    const bool nv_ok = (fmt == kNVFP4 && K % 64 == 0) || (fmt == kMXFP8 && K % 128 == 0);
    if (!nv_ok) return none;
    const bool f8 = fmt == kMXFP8;
    const int64_t nst = f8 ? K / 128 : (K + 127) / 128;   // the last NVFP4 stage may be half
    const int64_t tiles_nv = f8 ? ((M + 255) / 256) * ((N + 255) / 256) : ((M + 127) / 128) * ((N + 383) / 384);
    const int64_t min_units = f8 ? kSplitNvMinStagesPrefill / 2 : kSplitNvMinStagesPrefill;
    int64_t S = kSplitNvWorkgroups / tiles_nv;
    if (S > nst / min_units) S = nst / min_units;
    if (2 * tiles_nv > kSplitNvWorkgroups && !force) S = 1;
    if (force && S < 2 && nst >= 2) S = 2;
    if (S <= 1) return none;
    const int64_t per = (nst + S - 1) / S;
    S = (nst + per - 1) / per;
    if (S <= 1) return none;
    return SplitPlan{(int)S, (int)per, (size_t)(S * tiles * mt * 1024 * 4), true};
  }
  if (fmt == kNVFP4 && M > 64 && K % 64 == 0) {
    // NVFP4 with 3-4 M-tiles: the decode schedule converts every activation
    // fragment in every workgroup (1.25 fragments per MFMA); the 128 x 384
    // schedule converts 1/3 of one.  About one workgroup per CU along K.
    const int64_t nst = (K + 127) / 128, tiles_nv = (N + 383) / 384;
    int64_t S = kSplitNvWorkgroups / tiles_nv;
    if (S > nst / 2) S = nst / 2;
    if (!force && nst < 2 * kSplitMinSupersteps) S = 1;
    if (force && S < 2 && nst >= 2) S = 2;
    if (S > 1) {
      const int64_t per = (nst + S - 1) / S;
      S = (nst + per - 1) / per;
      if (S > 1) return SplitPlan{(int)S, (int)per, (size_t)(S * tiles * mt * 1024 * 4), true};
    }
  }
  int64_t S = (kSplitTargetWorkgroups + tiles - 1) / tiles;
  if (S > nss / 4) S = nss / 4;
  if (!force && nss < kSplitMinSupersteps) S = 1;
  if (force && S < 2 && nss >= 2) S = 2;
  if (S <= 1) return none;
  const int64_t per = (nss + S - 1) / S;
  S = (nss + per - 1) / per;
  return SplitPlan{(int)S, (int)per, (size_t)(S * tiles * mt * 1024 * 4), false};
}

int gemm_pick_variant(int64_t M, int64_t N, int64_t K, int fmt, int variant, size_t ws_bytes) {
  // fmt may be kMXFP8Mma (the split plan tells the two MXFP8 contractions apart)
  // NVFP4 rows of K % 32 == 16 elements: decode schedules only, any M (in
  // 128-row slices past 128 rows); an explicit prefill request is refused
  const bool half_k = fmt == kNVFP4 && (K / 2) % 16 != 0;
  if (variant == kVariantSplitK) {
    // the caller asked for split-K: a K of two supersteps (stages) at least;
    // above 128 rows NVFP4 with K % 64 == 0 or MXFP8 with K % 128 == 0
    if (M == 0 || N == 0) return kVariantSplitK;   // nothing to run
    return gemm_splitk_plan(M, N, K, fmt, true).splits > 1 ? kVariantSplitK : -1;
  }
  if (variant == -1) {
    const SplitPlan p = gemm_splitk_plan(M, N, K, fmt, false);
    if (p.splits > 1 && ws_bytes >= p.bytes) return kVariantSplitK;
  }
  if (half_k) return (variant == -1 || variant == 0) ? 0 : -1;
  if (variant == -1) return M <= 128 ? 0 : 1;
  if (variant == 0) return M <= 128 ? 0 : -1;   // the decode tile holds at most 128 tokens
  if (variant == 1) return 1;
  return -1;
}

hipError_t launch_gemm(const GemmArgs& g, int variant, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  switch (g.fmt) {
    case kNVFP4: return launch_fmt<kNVFP4>(g, variant, s);
    case kMXFP4: return launch_fmt<kMXFP4>(g, variant, s);
    case kMXFP8: return launch_fmt<kMXFP8>(g, variant, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lowbit
