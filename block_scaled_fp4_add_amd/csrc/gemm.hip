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
}  // namespace gk

namespace {
using gk::launch_fmt_epi;

template <int FMT>
hipError_t launch_fmt(const GemmArgs& g, int variant, hipStream_t s) {
  switch (g.epi) {
    case kEpiNone: return launch_fmt_epi<FMT, kEpiNone>(g, variant, s);
    case kEpiBias: return launch_fmt_epi<FMT, kEpiBias>(g, variant, s);
    case kEpiResidual: return launch_fmt_epi<FMT, kEpiResidual>(g, variant, s);
    case kEpiBiasResidual: return launch_fmt_epi<FMT, kEpiBiasResidual>(g, variant, s);
    case kEpiBiasGelu: return launch_fmt_epi<FMT, kEpiBiasGelu>(g, variant, s);
    case kEpiBiasGeluFp4: return launch_fmt_epi<FMT, kEpiBiasGeluFp4>(g, variant, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_pick_variant(int64_t M, int64_t N, int64_t K, int fmt, int variant) {
  (void)N;
  // NVFP4 rows of K % 32 == 16 elements: decode schedule only, any M (in
  // 128-row slices past 128 rows); an explicit prefill request is refused
  const bool half_k = fmt == kNVFP4 && (K / 2) % 16 != 0;
  if (half_k) return (variant == -1 || variant == 0) ? 0 : -1;
  if (variant == -1) return M <= 128 ? 0 : 1;
  if (variant == 0) return M <= 128 ? 0 : -1;   // the decode tile holds at most 128 tokens
  if (variant == 1) return 1;
  return -1;
}

hipError_t launch_gemm(const GemmArgs& g, int variant, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  return g.fmt == kMXFP4 ? launch_fmt<kMXFP4>(g, variant, s) : launch_fmt<kNVFP4>(g, variant, s);
}

}  // namespace lowbit
