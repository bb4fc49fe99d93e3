// gemm_inst_mx1.hip -- instantiates the GEMM launchers for MXFP4 with the
// Residual and BiasResidual epilogues (one compilation unit per pair).
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kMXFP4, kEpiResidual>(const GemmArgs& g, int variant, hipStream_t s);
template hipError_t launch_fmt_epi<kMXFP4, kEpiBiasResidual>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
