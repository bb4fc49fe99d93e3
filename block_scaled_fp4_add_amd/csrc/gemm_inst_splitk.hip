// gemm_inst_splitk.hip -- split-K launchers of the decode schedule for every
// (format, epilogue): the partial pass (one instantiation per format, M-tiles,
// waves and half-chunk flag, shared by the epilogues) and the reduce pass.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {

template <int FMT, int EPI, int MT, bool HALF>
hipError_t launch_splitk_mt(const GemmArgs& g, hipStream_t s) {
  // MXFP4 keeps two supersteps in flight per wave, NVFP4 (bound by its
  // dequantization work) one, as in the decode schedule
  constexpr bool DB = FMT == kMXFP4;
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
  const bool half = FMT == kNVFP4 && (g.K / 2) % 16 != 0;
#define LB_SPLIT(MT)                                                                        \
  if (mt == MT)                                                                             \
    return half ? launch_splitk_mt<FMT, EPI, MT, (FMT == kNVFP4)>(g, s)                   \
                : launch_splitk_mt<FMT, EPI, MT, false>(g, s);
  LB_SPLIT(1) LB_SPLIT(2) LB_SPLIT(3) LB_SPLIT(4)
#undef LB_SPLIT
  return hipErrorInvalidValue;
}

template hipError_t launch_splitk<kNVFP4, kEpiNone>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBias>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBiasResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBiasGelu>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kNVFP4, kEpiBiasGeluFp4>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiNone>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBias>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBiasResidual>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBiasGelu>(const GemmArgs& g, hipStream_t s);
template hipError_t launch_splitk<kMXFP4, kEpiBiasGeluFp4>(const GemmArgs& g, hipStream_t s);

}  // namespace gk
}  // namespace lowbit
