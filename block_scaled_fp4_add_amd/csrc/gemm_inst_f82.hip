// gemm_inst_f82.hip -- instantiates the GEMM launchers for MXFP8 operands with the
// BiasGelu and BiasGeluFp4 epilogues.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kMXFP8, kEpiBiasGelu>(const GemmArgs& g, int variant, hipStream_t s);
template hipError_t launch_fmt_epi<kMXFP8, kEpiBiasGeluFp4>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
