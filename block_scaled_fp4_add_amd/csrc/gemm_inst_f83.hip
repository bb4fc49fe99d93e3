// gemm_inst_f83.hip -- instantiates the GEMM launchers for MXFP8 operands with the
// FP8-output epilogue.
#include "gemm_kernels.hpp"

namespace lowbit {
namespace gk {
template hipError_t launch_fmt_epi<kMXFP8, kEpiFp8>(const GemmArgs& g, int variant, hipStream_t s);
}  // namespace gk
}  // namespace lowbit
