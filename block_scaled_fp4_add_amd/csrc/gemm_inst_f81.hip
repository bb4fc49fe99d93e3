// gemm_inst_f81.hip -- instantiates the GEMM launchers for MXFP8 operands with the
// Residual and BiasResidual epilogues.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kMXFP8, kEpiResidual>(const GemmArgs& g, int variant, hipStream_t s);
template hipError_t launch_fmt_epi<kMXFP8, kEpiBiasResidual>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
