// gemm_inst_mx2.hip -- instantiates the GEMM launchers for MXFP4 with the
// BiasGelu and BiasGeluFp4 epilogues (one compilation unit per pair).
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kMXFP4, kEpiBiasGelu>(const GemmArgs& g, int variant, hipStream_t s);
template hipError_t launch_fmt_epi<kMXFP4, kEpiBiasGeluFp4>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
