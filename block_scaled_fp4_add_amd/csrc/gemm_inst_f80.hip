// gemm_inst_f80.hip -- instantiates the GEMM launchers for MXFP8 operands with the
// None and Bias epilogues.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kMXFP8, kEpiNone>(const GemmArgs& g, int variant, hipStream_t s);
template hipError_t launch_fmt_epi<kMXFP8, kEpiBias>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
